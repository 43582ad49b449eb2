// C ABI of libdsp: validation, host geometry, device buffers and launches.
//
// Host geometry (data-only, recomputed per call): the solved frequency list,
// alias tables, 4 x 16 frequency tiles with their alias-slot unions, priors,
// the active bright-field set and the aberration polynomial.  Pages: "Where
// the 9 s of regularized preparation goes" (Code path: frequencies bucketed
// by alias count; prior; gather) and "Preparation in one kernel per alias
// count" (What changed 4: data-only layout computed once, kernels per optics).
#include "../../include/dsp.h"
#include "dsp_internal.hpp"
#include "dsp_kernels.hpp"

#include <hipfft/hipfft.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <tuple>
#include <vector>

using namespace dsp;

// Gram launch size: resident waves (from the kernel's occupancy) times this.
// Stream-K waves per resident wave slot.  More, shorter waves let the
// hardware's dispatch even out SIMDs that run at different speeds; past
// eight the partial-sum fixup costs more than the launches gain (whole
// full-frame step: 27.6 ms at 4, 27.2 at 8, 27.3 at 12 and at 16).
constexpr int GRAM_ROUNDS = 8;
static_assert(NOALLOC_SCRATCH_BYTES == DSP_NOALLOC_SCRATCH_BYTES, "one scratch size in the ABI and the kernels");

namespace {

thread_local std::string g_err;

dsp_status fail(dsp_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

#define HIP_TRY(expr)                                                                     \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess)                                                             \
            return fail(e_ == hipErrorOutOfMemory ? DSP_ENOMEM : DSP_EDEVICE, "%s: %s", #expr, \
                        hipGetErrorString(e_));                                           \
    } while (0)

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------

dsp_status check_scan(const dsp_scan *scan) {
    if (!scan) return fail(DSP_EINVAL, "scan is NULL");
    if (scan->n_scan < 4) return fail(DSP_EINVAL, "n_scan must be >= 4 (got %d)", scan->n_scan);
    if (scan->n_scan % 2) return fail(DSP_EUNSUPPORTED, "odd n_scan %d is not supported", scan->n_scan);
    if (scan->n_scan > 8192) return fail(DSP_EUNSUPPORTED, "n_scan %d above 8192", scan->n_scan);
    if (!(scan->step_A > 0.0) || !std::isfinite(scan->step_A)) return fail(DSP_EINVAL, "step_A must be > 0");
    return DSP_OK;
}

dsp_status check_optics(const dsp_optics *o) {
    if (!o) return fail(DSP_EINVAL, "optics is NULL");
    if (!(o->wavelength_A > 0.0) || !std::isfinite(o->wavelength_A)) return fail(DSP_EINVAL, "wavelength must be > 0");
    if (!(o->semiangle_rad > 0.0) || !std::isfinite(o->semiangle_rad)) return fail(DSP_EINVAL, "semiangle must be > 0");
    if (!(o->det_step_invA > 0.0) || !std::isfinite(o->det_step_invA)) return fail(DSP_EINVAL, "det_step must be > 0");
    if (o->soft_aperture != 0 && o->soft_aperture != 1) return fail(DSP_EINVAL, "soft_aperture must be 0 or 1");
    if (!(o->depth_A >= 0.0) || !std::isfinite(o->depth_A)) return fail(DSP_EINVAL, "depth_A must be finite and >= 0");
    if (!std::isfinite(o->tilt_rad[0]) || !std::isfinite(o->tilt_rad[1])) return fail(DSP_EINVAL, "tilt not finite");
    if (o->n_aber < 0 || o->n_aber > DSP_MAX_ABERRATIONS)
        return fail(DSP_EINVAL, "n_aber %d outside [0, %d]", o->n_aber, DSP_MAX_ABERRATIONS);
    for (int i = 0; i < o->n_aber; ++i) {
        const dsp_aberration &a = o->aber[i];
        if (a.n < 1 || a.n > 5 || a.m < 0 || a.m > a.n + 1 || ((a.n + 1 - a.m) & 1))
            return fail(DSP_EINVAL, "aberration %d: (n, m) = (%d, %d) is not a Krivanek term of order 1..5", i, a.n, a.m);
        if (!std::isfinite(a.c_A) || !std::isfinite(a.phi_rad)) return fail(DSP_EINVAL, "aberration %d not finite", i);
    }
    return DSP_OK;
}

dsp_status check_upsampling(int u) {
    if (u < 1) return fail(DSP_EINVAL, "upsampling must be >= 1 (got %d)", u);
    if (u > 4) return fail(DSP_EUNSUPPORTED, "upsampling %d above 4", u);
    return DSP_OK;
}

// ---------------------------------------------------------------------------
// optics helpers
// ---------------------------------------------------------------------------

double binom(int n, int k) {
    double r = 1.0;
    for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
    return r;
}

// chi(theta) polynomial coefficients (rad) from the Krivanek terms:
// t^(n+1) cos(m (p - phi)) = Re[exp(-i m phi) w^m] (w w*)^((n+1-m)/2),
// w^m = sum_k C(m,k) i^k tx^(m-k) ty^k, (w w*)^h = sum_l C(h,l) tx^(2h-2l) ty^(2l).
void chi_coefficients(const dsp_optics *o, double *coef) {
    for (int i = 0; i < CHI_NCOEF; ++i) coef[i] = 0.0;
    const double two_pi = 6.283185307179586476925286766559;
    for (int t = 0; t < o->n_aber; ++t) {
        const dsp_aberration &a = o->aber[t];
        const int n = a.n, m = a.m, h = (n + 1 - m) / 2;
        const double f = two_pi / o->wavelength_A * a.c_A / (n + 1);
        const double cm = std::cos(m * a.phi_rad), sm = std::sin(m * a.phi_rad);
        for (int k = 0; k <= m; ++k) {
            // Re[(cm - i sm) i^k] = cm Re(i^k) + sm Im(i^k)
            static const int re_ik[4] = {1, 0, -1, 0};
            static const int im_ik[4] = {0, 1, 0, -1};
            const double ck = binom(m, k) * (cm * re_ik[k & 3] + sm * im_ik[k & 3]);
            if (ck == 0.0) continue;
            for (int l = 0; l <= h; ++l) {
                const int px = (m - k) + 2 * (h - l);
                const int py = k + 2 * l;
                coef[chi_off(py) + px] += f * ck * binom(h, l);
            }
        }
    }
}

OpticsDev make_optics_dev(const dsp_optics *o) {
    OpticsDev d;
    d.lam = o->wavelength_A;
    d.tau_y = o->tilt_rad[0];
    d.tau_x = o->tilt_rad[1];
    d.pt2 = M_PI * o->depth_A / (2.0 * o->wavelength_A);
    chi_coefficients(o, d.chi_c);
    return d;
}

ApertureDev make_aperture_dev(const dsp_optics *o) {
    ApertureDev a;
    a.kc = o->semiangle_rad / o->wavelength_A;
    a.inv_dk = 1.0 / o->det_step_invA;
    a.soft = o->soft_aperture;
    const double h = 0.5 * o->det_step_invA;
    if (a.soft) {
        const double rin = std::max(0.0, a.kc - h);
        a.rin2 = rin * rin;
        a.rout2 = (a.kc + h) * (a.kc + h);
        a.rlim2 = a.rout2;
    } else {
        a.rin2 = a.kc * a.kc;
        a.rout2 = a.kc * a.kc;
        a.rlim2 = std::nextafter(a.rout2, HUGE_VAL);   // d2 <= kc^2  <=>  d2 < next double
    }
    const double lam = o->wavelength_A;
    a.lrlim2 = lam * lam * a.rlim2;
    a.lrin2 = lam * lam * a.rin2;
    a.lkc = o->semiangle_rad;                      // lambda (alpha / lambda)
    a.inv_ldk = 1.0 / (lam * o->det_step_invA);
    return a;
}

// a(|k|) > 0, evaluated as the definition: clamp(1/2 + (kc - |k|)/dk, 0, 1).
bool pixel_active(const dsp_optics *o, double ky, double kx) {
    const double kabs = std::hypot(ky, kx);
    const double kc = o->semiangle_rad / o->wavelength_A;
    if (o->soft_aperture) {
        double a = 0.5 + (kc - kabs) / o->det_step_invA;
        a = std::min(1.0, std::max(0.0, a));
        return a > 0.0;
    }
    return kabs <= kc;
}

double alias_radius(const dsp_optics *o) {
    double r = (2.0 * o->semiangle_rad) / o->wavelength_A;
    if (o->soft_aperture) r = r + o->det_step_invA;
    return r;
}

// ---------------------------------------------------------------------------
// frequency geometry
// ---------------------------------------------------------------------------

struct Geometry {
    int N = 0, u = 0, n_q = 0, a_max = 0;
    double dq = 0.0;
    std::vector<int32_t> q;       // [n_q][2] stored (iy, ix)
    std::vector<int32_t> count;   // [n_q]
    std::vector<int32_t> K;       // [n_q][a_max][2]
    std::vector<int32_t> jy, jx;  // [n_q][a_max] alias offsets
    int hist[10] = {0};
};

dsp_status build_geometry(const dsp_scan *scan, const dsp_optics *o, int u, Geometry &g) {
    const int N = scan->n_scan;
    g.N = N;
    g.u = u;
    g.dq = 1.0 / (N * scan->step_A);
    const double dq = g.dq;
    const double R = alias_radius(o);
    const int half = (u * N) / 2;
    std::vector<int32_t> ktmp;
    std::vector<int32_t> jtmp;
    std::vector<int> cnt;
    g.q.clear();
    const int maxc = (2 * u + 1) * (2 * u + 1);
    for (int iy = 0; iy < N; ++iy) {
        if (iy == N / 2) continue;
        const int yh = iy < N / 2 ? iy : iy - N;
        for (int ix = 0; ix < N / 2; ++ix) {
            if (ix == 0 && yh <= 0) continue;
            g.q.push_back(iy);
            g.q.push_back(ix);
            int c = 0;
            for (int jyy = -u; jyy <= u; ++jyy) {
                const int ky = yh + jyy * N;
                if (ky < -half || ky >= half) continue;
                for (int jxx = -u; jxx <= u; ++jxx) {
                    const int kx = ix + jxx * N;
                    if (kx < -half || kx >= half) continue;
                    const double k2 = (double)((long long)ky * ky + (long long)kx * kx);
                    if (k2 * (dq * dq) < R * R) {
                        ktmp.push_back(ky);
                        ktmp.push_back(kx);
                        jtmp.push_back(jyy);
                        jtmp.push_back(jxx);
                        ++c;
                    }
                }
            }
            (void)maxc;
            cnt.push_back(c);
        }
    }
    g.n_q = (int)cnt.size();
    g.a_max = 0;
    for (int c : cnt) g.a_max = std::max(g.a_max, c);
    if (g.a_max > 9) return fail(DSP_EALIAS, "alias count %d above 9", g.a_max);
    g.count.assign(cnt.begin(), cnt.end());
    const int am = std::max(1, g.a_max);
    g.K.assign((size_t)g.n_q * am * 2, 0);
    g.jy.assign((size_t)g.n_q * am, 0);
    g.jx.assign((size_t)g.n_q * am, 0);
    size_t pos = 0;
    for (int i = 0; i < g.n_q; ++i) {
        for (int m = 0; m < cnt[i]; ++m, ++pos) {
            g.K[((size_t)i * am + m) * 2] = ktmp[2 * pos];
            g.K[((size_t)i * am + m) * 2 + 1] = ktmp[2 * pos + 1];
            g.jy[(size_t)i * am + m] = jtmp[2 * pos];
            g.jx[(size_t)i * am + m] = jtmp[2 * pos + 1];
        }
        g.hist[std::min(cnt[i], 9)]++;
    }
    return DSP_OK;
}

// Lane groups of at most 64 scan frequencies, cut along G's 128-byte lines.
// Row yh (stored row iy = yh mod N) starts at element iy nh of a plane, so its
// first line boundary lies at column h = (-iy nh) mod 16.  Its columns
// [0, ncol) split into runs that each fill part of one line: the head [0, h)
// is block 0 and the run starting at column h + 16 (b - 1) is block b.  Within
// a block the runs of consecutive rows, cut down to the columns `keep`
// accepts, are packed in row order into groups of at most 64 lanes, spanning
// at most `max_rows` rows; a run is never split, so each line feeds one group.
typedef std::vector<std::pair<int16_t, int16_t>> Lanes;   // (yh, ix) per lane

template <class Keep>
std::vector<Lanes> pack_line_runs(int N, int nh, int yh_lo, int yh_hi, int ncol, int max_rows, Keep keep) {
    std::vector<Lanes> out;
    const int n_blk = 2 + (ncol - 1) / LINE_X;
    Lanes cur, run;
    int cur_row0 = 0;
    for (int b = 0; b < n_blk; ++b) {
        for (int yh = yh_lo; yh <= yh_hi; ++yh) {
            const long long iy = yh < 0 ? yh + N : yh;
            const int h = (int)((LINE_X - (iy * nh) % LINE_X) % LINE_X);
            const int c0 = b == 0 ? 0 : h + LINE_X * (b - 1);
            const int c1 = std::min(ncol, b == 0 ? h : c0 + LINE_X);
            run.clear();
            for (int ix = c0; ix < c1; ++ix)
                if (keep(yh, ix)) run.emplace_back((int16_t)yh, (int16_t)ix);
            if (run.empty()) continue;
            if (!cur.empty() && (cur.size() + run.size() > 64 || yh - cur_row0 >= max_rows)) {
                out.push_back(cur);
                cur.clear();
            }
            if (cur.empty()) cur_row0 = yh;
            cur.insert(cur.end(), run.begin(), run.end());
        }
        if (!cur.empty()) {
            out.push_back(cur);
            cur.clear();
        }
    }
    return out;
}

// Group the solved frequencies into lane groups (pack_line_runs) and collect
// each tile's sorted union of alias offsets.  A tile whose union exceeds the
// kernels' slot maximum is split into sub-tiles with disjoint lane subsets
// (greedy over the lanes' alias sets).
struct TileGroups {
    std::vector<GramTile> tiles;      // grouped by nj, groups in ascending nj
    std::vector<int> group_nj, group_off, group_n;
};

typedef std::vector<std::pair<int, int>> JSet;

void finish_tile(GramTile &t, const JSet &js_in, const Geometry &g,
                 std::map<int, std::vector<std::pair<long long, GramTile>>> &by_nj) {
    const int am = std::max(1, g.a_max);
    JSet js = js_in;
    if (js.empty()) js.emplace_back(0, 0);   // no aliases anywhere: one inactive slot
    t.nj = (int)js.size();
    long long cost = 0;
    for (int s = 0; s < t.nj; ++s) {
        t.jy[s] = (int8_t)js[s].first;
        t.jx[s] = (int8_t)js[s].second;
    }
    double sy = 0.0, sx = 0.0;
    int nv = 0;
    for (int l = 0; l < 64; ++l) {
        const int qi = t.qidx[l];
        t.mask[l] = 0;
        if (qi < 0) continue;
        sy += t.lyh[l];
        sx += t.lix[l];
        ++nv;
        cost += g.count[qi];
        unsigned msk = 0;
        for (int m = 0; m < g.count[qi]; ++m) {
            const std::pair<int, int> j(g.jy[(size_t)qi * am + m], g.jx[(size_t)qi * am + m]);
            const int s = (int)(std::lower_bound(js.begin(), js.end(), j) - js.begin());
            msk |= 1u << s;
        }
        t.mask[l] = (uint16_t)msk;
    }
    t.cy = (float)(nv ? sy / nv : 0.0);
    t.cx = (float)(nv ? sx / nv : 0.0);
    // radius of the valid lanes about the stored centre, for the kernels'
    // per-pixel slot test (a bound: rounded up and widened by a part in 1e6)
    double rad = 0.0;
    for (int l = 0; l < 64; ++l) {
        if (t.qidx[l] < 0) continue;
        rad = std::max(rad, std::hypot((double)t.lyh[l] - (double)t.cy, (double)t.lix[l] - (double)t.cx));
    }
    t.rad = std::nextafter((float)(rad * (1.0 + 1e-6)), INFINITY);
    by_nj[t.nj].emplace_back(-cost, t);
}

dsp_status build_gram_tiles(const Geometry &g, int max_nj, TileGroups &tg) {
    const int N = g.N, am = std::max(1, g.a_max);
    // index of each solved frequency by (iy, ix)
    std::vector<int32_t> qidx((size_t)N * (N / 2), -1);
    for (int i = 0; i < g.n_q; ++i) qidx[(size_t)g.q[2 * i] * (N / 2) + g.q[2 * i + 1]] = i;
    std::map<int, std::vector<std::pair<long long, GramTile>>> by_nj;
    const int nh = N / 2 + 1;
    // rows -N/2+1 .. N/2-1 and columns 0 .. N/2-1: the solved half-plane
    // leaves out the Nyquist row and column
    auto solved = [&](int yh, int ix) { return qidx[(size_t)(yh < 0 ? yh + N : yh) * (N / 2) + ix] >= 0; };
    const std::vector<Lanes> groups = pack_line_runs(N, nh, -N / 2 + 1, N / 2 - 1, N / 2, 8, solved);
    for (const Lanes &grp : groups) {
        int lane_q[64];
        JSet lane_js[64];
        JSet uni;
        int nvalid = 0;
        GramTile base;
        std::memset(&base, 0, sizeof base);
        for (int l = 0; l < 64; ++l) {
            lane_q[l] = -1;
            if (l >= (int)grp.size()) continue;
            const int yh = grp[l].first, ix = grp[l].second;
            base.lyh[l] = (int16_t)yh;
            base.lix[l] = (int16_t)ix;
            const int qi = qidx[(size_t)(yh < 0 ? yh + N : yh) * (N / 2) + ix];
            lane_q[l] = qi;
            ++nvalid;
            for (int m = 0; m < g.count[qi]; ++m)
                lane_js[l].emplace_back(g.jy[(size_t)qi * am + m], g.jx[(size_t)qi * am + m]);
            uni.insert(uni.end(), lane_js[l].begin(), lane_js[l].end());
        }
        if (nvalid == 0) continue;
        std::sort(uni.begin(), uni.end());
        uni.erase(std::unique(uni.begin(), uni.end()), uni.end());
        if ((int)uni.size() <= max_nj) {
            for (int l = 0; l < 64; ++l) base.qidx[l] = lane_q[l];
            finish_tile(base, uni, g, by_nj);
            continue;
        }
        // split: each sub-tile takes lanes while its union stays within max_nj
        bool taken[64] = {false};
        int left = nvalid;
        while (left > 0) {
            GramTile t = base;
            JSet js;
            for (int l = 0; l < 64; ++l) t.qidx[l] = -1;
            for (int l = 0; l < 64; ++l) {
                if (lane_q[l] < 0 || taken[l]) continue;
                JSet tryu = js;
                tryu.insert(tryu.end(), lane_js[l].begin(), lane_js[l].end());
                std::sort(tryu.begin(), tryu.end());
                tryu.erase(std::unique(tryu.begin(), tryu.end()), tryu.end());
                if ((int)tryu.size() > max_nj) continue;
                js.swap(tryu);
                t.qidx[l] = lane_q[l];
                taken[l] = true;
                --left;
            }
            if (js.empty() && left > 0) {
                // a single frequency above the maximum (checked by the caller)
                return fail(DSP_EALIAS, "a frequency needs more than %d alias slots", max_nj);
            }
            finish_tile(t, js, g, by_nj);
        }
    }
    tg.tiles.clear();
    tg.group_nj.clear();
    tg.group_off.clear();
    tg.group_n.clear();
    for (auto &kv : by_nj) {
        auto &v = kv.second;
        std::stable_sort(v.begin(), v.end(), [](const std::pair<long long, GramTile> &a,
                                                const std::pair<long long, GramTile> &b) { return a.first < b.first; });
        tg.group_nj.push_back(kv.first);
        tg.group_off.push_back((int)tg.tiles.size());
        tg.group_n.push_back((int)v.size());
        for (auto &p : v) tg.tiles.push_back(p.second);
    }
    return DSP_OK;
}

struct ActiveSet {
    std::vector<int32_t> idx;
    std::vector<PixelBase> pix;
    std::vector<long long> goff;   // element offset of each active pixel's plane in G
    double scale = 0.0;
};

dsp_status build_active(const double *k, const double *w, int n_bf, const dsp_optics *o, int N, ActiveSet &as) {
    as.idx.clear();
    as.pix.clear();
    as.goff.clear();
    as.scale = 0.0;
    const long long plane = (long long)N * (N / 2 + 1);
    for (int i = 0; i < n_bf; ++i) {
        const double ky = k[2 * i], kx = k[2 * i + 1];
        if (!std::isfinite(ky) || !std::isfinite(kx)) return fail(DSP_EINVAL, "bf_coords[%d] not finite", i);
        const double wi = w ? w[i] : 1.0;
        if (!(wi >= 0.0) || !std::isfinite(wi)) return fail(DSP_EINVAL, "weights[%d] must be finite and >= 0", i);
        if (!pixel_active(o, ky, kx)) continue;
        PixelBase p;
        p.ky = ky;
        p.kx = kx;
        p.w = wi;
        p.sw = std::sqrt(wi);
        as.idx.push_back(i);
        as.pix.push_back(p);
        as.goff.push_back((long long)i * plane);
        as.scale += wi;
    }
    return DSP_OK;
}

// ---------------------------------------------------------------------------
// stream-K plan of one Gram launch
// ---------------------------------------------------------------------------
struct StreamKPlan {
    std::vector<long long> wbegin;   // [W + 1]
    std::vector<int> seg_off;        // [W]
    std::vector<int> seg_first;      // [T + 1]
    int n_segs = 0;
};

// Runs work(t0, t1) over [0, nt) split among up to 16 threads; a range whose
// thread cannot be started runs on the calling thread.
template <class F>
void parallel_tiles(int nt, const F &work) {
    const int nth = std::max(1, std::min<int>({16, (int)std::thread::hardware_concurrency(), nt / 16 + 1}));
    std::vector<std::thread> th;
    for (int i = 1; i < nth; ++i) {
        const int t0 = (int)((long long)nt * i / nth), t1 = (int)((long long)nt * (i + 1) / nth);
        try {
            th.emplace_back(work, t0, t1);
        } catch (...) {
            work(t0, t1);
        }
    }
    work(0, (int)((long long)nt / nth));
    for (auto &x : th) x.join();
}

// Estimated cost of every (tile, pixel) iteration of one Gram launch, in
// units of about four instructions: a fixed part per pixel, and per slot
// the kernels' own reach test (tile centre and radius): a slot that may
// have a lobe in support costs its support tests, each admitted lobe an
// evaluation.  Tile-major, n_pix per tile; threads split the tiles.
void gram_iteration_costs(const GramTile *tiles, int nt, const std::vector<PixelBase> &pix, const Geometry &g,
                          double ra, std::vector<uint16_t> &cost) {
    // C_PIX covers the pixel's G load and power term as well as its
    // instructions (measured: 8 and 32 bracket the best plans)
    constexpr int C_PIX = 16, C_SLOT = 3, C_LOBE = 20;
    const int n_pix = (int)pix.size();
    cost.assign((size_t)nt * n_pix, 0);
    auto work = [&](int t0, int t1) {
        for (int t = t0; t < t1; ++t) {
            const GramTile &tl = tiles[t];
            unsigned used = 0;
            for (int l = 0; l < 64; ++l)
                if (tl.qidx[l] >= 0) used |= tl.mask[l];
            double cy[MAX_SLOTS], cx[MAX_SLOTS];
            for (int s = 0; s < tl.nj; ++s) {
                cy[s] = ((double)tl.cy + (double)tl.jy[s] * g.N) * g.dq;
                cx[s] = ((double)tl.cx + (double)tl.jx[s] * g.N) * g.dq;
            }
            const double rr = ra + (double)tl.rad * g.dq;
            const double thr = rr * rr;
            uint16_t *c = cost.data() + (size_t)t * n_pix;
            for (int p = 0; p < n_pix; ++p) {
                const double ky = pix[p].ky, kx = pix[p].kx;
                int v = C_PIX;
                for (int s = 0; s < tl.nj; ++s) {
                    if (!((used >> s) & 1u)) continue;
                    const double ly = ky - cy[s], lx = kx - cx[s], ry = ky + cy[s], rx = kx + cx[s];
                    const int nl = (ly * ly + lx * lx < thr) + (ry * ry + rx * rx < thr);
                    if (nl) v += C_SLOT + C_LOBE * nl;
                }
                c[p] = (uint16_t)v;
            }
        }
    };
    parallel_tiles(nt, work);
}

// Split the tiles x pixels iteration space into n_waves contiguous ranges of
// equal estimated cost (per-iteration costs, tile-major), then number each
// wave's tile segments.
template <class Cost>
void plan_stream_k_iter(const Cost &cost, int T, int n_pix, int n_waves, StreamKPlan &pl) {
    const long long total_it = (long long)T * n_pix;
    unsigned long long total = 0;
    for (long long i = 0; i < total_it; ++i) total += cost[i];
    const int W = n_waves;
    pl.wbegin.assign(W + 1, total_it);
    pl.wbegin[0] = 0;
    unsigned long long acc = 0;
    int w = 1;
    for (long long i = 0; i < total_it && w < W; ++i) {
        acc += cost[i];
        // boundary w after the iteration where the running cost reaches w / W
        while (w < W && acc * (unsigned long long)W >= total * (unsigned long long)w) pl.wbegin[w++] = i + 1;
    }
    pl.seg_off.assign(W, 0);
    pl.seg_first.assign(T + 1, -1);
    int ns = 0;
    for (int ww = 0; ww < W; ++ww) {
        pl.seg_off[ww] = ns;
        long long it = pl.wbegin[ww];
        const long long e = pl.wbegin[ww + 1];
        while (it < e) {
            const int tt = (int)(it / n_pix);
            if (pl.seg_first[tt] < 0) pl.seg_first[tt] = ns;
            it = std::min(e, (long long)(tt + 1) * n_pix);
            ++ns;
        }
    }
    pl.seg_first[T] = ns;
    pl.n_segs = ns;
}

// Reach bits of every (SSB tile, pixel) iteration, as the one-set SSB kernel
// tests them (tile centre and radius): bit 0 when the L lobe may be in
// support for some lane, bit 1 the R lobe.  Tile-major; threads split the
// tiles.
void ssb_reach_bits(const std::vector<SsbTile> &tiles, const std::vector<PixelBase> &pix, double dq, double ra,
                    std::vector<uint8_t> &bits) {
    const int nt = (int)tiles.size(), n_pix = (int)pix.size();
    bits.assign((size_t)nt * n_pix, 0);
    auto work = [&](int t0, int t1) {
        for (int t = t0; t < t1; ++t) {
            const SsbTile &tl = tiles[t];
            const double cy = (double)tl.cy * dq, cx = (double)tl.cx * dq;
            const double rr = ra + (double)tl.rad * dq, thr = rr * rr;
            uint8_t *b = bits.data() + (size_t)t * n_pix;
            for (int p = 0; p < n_pix; ++p) {
                const double ly = pix[p].ky - cy, lx = pix[p].kx - cx, ry = pix[p].ky + cy, rx = pix[p].kx + cx;
                b[p] = (uint8_t)((ly * ly + lx * lx < thr ? 1 : 0) | (ry * ry + rx * rx < thr ? 2 : 0));
            }
        }
    };
    parallel_tiles(nt, work);
}

// (cos, sin)(j pi / 128), j = 0..255, rounded from long double.
void trig_table_host(double2 *T) {
    const long double pi = 3.141592653589793238462643383279502884L;
    for (int j = 0; j < TRIG_N; ++j) {
        const long double a = pi * j / 128.0L;
        T[j] = make_double2((double)std::cos(a), (double)std::sin(a));
    }
}

// The table on a device: uploaded once per device, kept until the process ends.
dsp_status trig_table_device(int device, const double2 **out) {
    static std::mutex mu;
    static std::map<int, double2 *> tables;
    std::lock_guard<std::mutex> lock(mu);
    auto f = tables.find(device);
    if (f != tables.end()) {
        *out = f->second;
        return DSP_OK;
    }
    double2 host[TRIG_N];
    trig_table_host(host);
    double2 *d = nullptr;
    HIP_TRY(hipMalloc((void **)&d, sizeof host));
    HIP_TRY(hipMemcpy(d, host, sizeof host, hipMemcpyHostToDevice));
    tables[device] = d;
    *out = d;
    return DSP_OK;
}

// atan(i/64), i = 0..ATAN_N - 1 (atan2_tab), rounded from long double.
void atan_table_host(double *A) {
    for (int i = 0; i < ATAN_N; ++i) A[i] = (double)atanl((long double)i / 64.0L);
}

// The atan table on a device: uploaded once per device, kept until the
// process ends.
dsp_status atan_table_device(int device, const double **out) {
    static std::mutex mu;
    static std::map<int, double *> tables;
    std::lock_guard<std::mutex> lock(mu);
    auto f = tables.find(device);
    if (f != tables.end()) {
        *out = f->second;
        return DSP_OK;
    }
    double host[ATAN_N];
    atan_table_host(host);
    double *d = nullptr;
    HIP_TRY(hipMalloc((void **)&d, sizeof host));
    HIP_TRY(hipMemcpy(d, host, sizeof host, hipMemcpyHostToDevice));
    tables[device] = d;
    *out = d;
    return DSP_OK;
}

// e^{+2 pi i m / N} for m < N/2 (the fused loss transforms), from long
// double on the host, one device table per (device, N) kept for the process.
dsp_status twiddle_table_device(int device, int N, const double2 **out) {
    static std::mutex mu;
    static std::map<std::pair<int, int>, double2 *> tables;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(device, N);
    auto f = tables.find(key);
    if (f != tables.end()) {
        *out = f->second;
        return DSP_OK;
    }
    std::vector<double2> host((size_t)N / 2);
    const long double two_pi = 6.283185307179586476925286766559005768L;
    for (int m = 0; m < N / 2; ++m) {
        const long double a = two_pi * (long double)m / (long double)N;
        host[(size_t)m] = make_double2((double)cosl(a), (double)sinl(a));
    }
    double2 *d = nullptr;
    HIP_TRY(hipMalloc((void **)&d, host.size() * sizeof(double2)));
    HIP_TRY(hipMemcpy(d, host.data(), host.size() * sizeof(double2), hipMemcpyHostToDevice));
    tables[key] = d;
    *out = d;
    return DSP_OK;
}

// Scratch memory per (device, stream) for temporaries that live within one
// call (Gram partial sums, SSB per-call tables).  Work on one stream runs in
// order, so consecutive calls can reuse the same bytes; the arena only grows
// (hipFree of the old block waits for the device first).  Kept until the
// process ends.
struct Arena {
    int device;
    hipStream_t stream;
    char *ptr;
    size_t size;
};

dsp_status arena_get(int device, hipStream_t stream, size_t bytes, char **out) {
    static std::mutex mu;
    static std::vector<Arena> arenas;
    std::lock_guard<std::mutex> lock(mu);
    bytes = std::max<size_t>(bytes, 256);
    for (auto &a : arenas) {
        if (a.device != device || a.stream != stream) continue;
        if (a.size < bytes) {
            const size_t grow = std::max(bytes, a.size + a.size / 2);
            HIP_TRY(hipFree(a.ptr));   // waits for the device before freeing
            a.ptr = nullptr;
            a.size = 0;
            HIP_TRY(hipMalloc((void **)&a.ptr, grow));
            a.size = grow;
        }
        *out = a.ptr;
        return DSP_OK;
    }
    Arena a{device, stream, nullptr, bytes};
    HIP_TRY(hipMalloc((void **)&a.ptr, bytes));
    arenas.push_back(a);
    *out = a.ptr;
    return DSP_OK;
}

// Carves aligned pieces out of one arena block.
struct Carve {
    char *base;
    size_t off = 0;
    template <class T>
    T *take(size_t n) {
        T *p = (T *)(base + off);
        off += (n * sizeof(T) + 255) / 256 * 256;
        return p;
    }
};
inline size_t carve_size(size_t n, size_t elem) { return (n * elem + 255) / 256 * 256; }

// Per-device cache of handle buffers.  A destroyed handle's buffers are
// kept, each with the events of the last work queued with them on every
// stream the handle ran on; a later request that fits a kept block takes it
// after making its own stream wait on those events.  Neither the release
// nor the reuse waits on the host, and repeated prepares of one workload
// allocate nothing.  Sizes are rounded up to 2 MiB; a request takes the
// smallest kept block of at least its size and at most twice it.  Above
// 4 GiB kept per device the oldest blocks are freed (after their events).
// Events that a reuse has waited on are destroyed once they have completed.
struct PoolBlock {
    void *ptr;
    size_t bytes;
    std::vector<hipEvent_t> ev;
};
struct DevicePool {
    int device;
    std::vector<PoolBlock> kept;      // oldest first
    std::vector<hipEvent_t> retired;  // waited on; destroyed once complete
    size_t bytes = 0;
};
constexpr size_t kPoolCap = size_t(4) << 30;
constexpr size_t kPoolGrain = size_t(2) << 20;
std::mutex g_pool_mu;
std::vector<DevicePool> g_pools;

DevicePool &pool_of(int device) {
    for (auto &p : g_pools)
        if (p.device == device) return p;
    g_pools.push_back(DevicePool{device, {}, {}, 0});
    return g_pools.back();
}

void pool_sweep(DevicePool &P) {
    size_t j = 0;
    for (size_t i = 0; i < P.retired.size(); ++i) {
        if (hipEventQuery(P.retired[i]) == hipSuccess)
            (void)hipEventDestroy(P.retired[i]);
        else
            P.retired[j++] = P.retired[i];
    }
    P.retired.resize(j);
}

// Frees every kept block of the device (after its events); the caller holds
// the lock and has made the device current.
void pool_drain(DevicePool &P) {
    for (auto &b : P.kept) {
        for (auto e : b.ev) {
            (void)hipEventSynchronize(e);
            (void)hipEventDestroy(e);
        }
        (void)hipFree(b.ptr);
    }
    P.kept.clear();
    P.bytes = 0;
}

// The device must be current.
dsp_status pool_alloc(int device, hipStream_t stream, size_t bytes, void **out) {
    *out = nullptr;
    bytes = (std::max<size_t>(bytes, 1) + kPoolGrain - 1) / kPoolGrain * kPoolGrain;
    PoolBlock blk{nullptr, 0, {}};
    {
        std::lock_guard<std::mutex> lock(g_pool_mu);
        DevicePool &P = pool_of(device);
        pool_sweep(P);
        int best = -1;
        for (int i = 0; i < (int)P.kept.size(); ++i) {
            const size_t b = P.kept[i].bytes;
            if (b >= bytes && b <= 2 * bytes && (best < 0 || b < P.kept[best].bytes)) best = i;
        }
        if (best >= 0) {
            blk = P.kept[best];
            P.kept.erase(P.kept.begin() + best);
            P.bytes -= blk.bytes;
            // every event is retired, also those after a failed wait
            hipError_t err = hipSuccess;
            for (auto e : blk.ev) {
                if (err == hipSuccess) err = hipStreamWaitEvent(stream, e, 0);
                P.retired.push_back(e);
            }
            if (err != hipSuccess) {
                (void)hipFree(blk.ptr);
                return fail(DSP_EDEVICE, "hipStreamWaitEvent: %s", hipGetErrorString(err));
            }
            *out = blk.ptr;
            return DSP_OK;
        }
    }
    hipError_t err = hipMalloc(out, bytes);
    if (err == hipErrorOutOfMemory) {
        // give the kept blocks back and try once more
        (void)hipGetLastError();
        {
            std::lock_guard<std::mutex> lock(g_pool_mu);
            pool_drain(pool_of(device));
        }
        err = hipMalloc(out, bytes);
    }
    if (err != hipSuccess) {
        *out = nullptr;
        return fail(err == hipErrorOutOfMemory ? DSP_ENOMEM : DSP_EDEVICE, "hipMalloc(%zu): %s", bytes,
                    hipGetErrorString(err));
    }
    return DSP_OK;
}

// Keeps a block for reuse once the events (moved in) have completed.  The
// device must be current.
void pool_release(int device, void *ptr, size_t bytes, std::vector<hipEvent_t> ev) {
    if (!ptr) {
        for (auto e : ev) (void)hipEventDestroy(e);
        return;
    }
    bytes = (std::max<size_t>(bytes, 1) + kPoolGrain - 1) / kPoolGrain * kPoolGrain;
    std::lock_guard<std::mutex> lock(g_pool_mu);
    DevicePool &P = pool_of(device);
    P.kept.push_back(PoolBlock{ptr, bytes, std::move(ev)});
    P.bytes += bytes;
    while (P.bytes > kPoolCap && !P.kept.empty()) {
        PoolBlock b = P.kept.front();
        P.kept.erase(P.kept.begin());
        P.bytes -= b.bytes;
        for (auto e : b.ev) {
            (void)hipEventSynchronize(e);
            (void)hipEventDestroy(e);
        }
        (void)hipFree(b.ptr);
    }
}

double now_ms() {
    using namespace std::chrono;
    return duration<double, std::milli>(steady_clock::now().time_since_epoch()).count();
}

template <class T>
dsp_status dev_alloc(T **p, size_t n) {
    *p = nullptr;
    if (n == 0) n = 1;
    HIP_TRY(hipMalloc((void **)p, n * sizeof(T)));
    return DSP_OK;
}



// ---------------------------------------------------------------------------
// data-only layout, cached across prepares
// ---------------------------------------------------------------------------
// Everything a prepare needs that does not depend on the aberrations or the
// data values: frequencies, aliases, tiles, priors, alias-count buckets,
// active pixels and their weights, the stream-K plans, and device copies
// ("Preparation in one kernel per alias count", What changed 4: a data-only
// layout computed once per data, sampling and prior).  Keyed by device,
// scan, aperture, upsampling, method, prior, and the exact bright-field
// coordinates and weights.
struct LayoutKey {
    int device = 0, n_scan = 0, u = 0, method = 0, soft = 0, n_bf = 0;
    double step = 0, lam = 0, alpha = 0, dk = 0, smooth = 0;
    std::vector<double> coords, weights;   // weights empty when NULL
    bool operator==(const LayoutKey &o) const {
        return device == o.device && n_scan == o.n_scan && u == o.u && method == o.method && soft == o.soft &&
               n_bf == o.n_bf && step == o.step && lam == o.lam && alpha == o.alpha && dk == o.dk &&
               smooth == o.smooth && coords == o.coords && weights == o.weights;
    }
};

struct Layout {
    LayoutKey key;
    Geometry geo;
    TileGroups tg;
    ActiveSet act;
    std::vector<int> bucket_off, bucket_n;
    std::vector<int32_t> bucket;
    std::vector<double> prior;
    std::vector<int> sk_waves;                // waves of each group's Gram launch
    std::vector<size_t> wb_off, so_off, sf_off;
    std::vector<long long> sk_wbegin;         // stream-K tables of all groups
    std::vector<int> sk_int;
    size_t max_partial = 0;                   // doubles of the largest group's partial sums
    double host_ms = 0.0;                     // time to build
    // device copies
    PixelBase *d_pixbase = nullptr;           // active pixels: k and weights
    long long *d_goff = nullptr;              // their plane offsets in G
    GramTile *d_tiles = nullptr;
    double *d_prior = nullptr;                // [n_q][a_max]
    int32_t *d_count = nullptr;               // [n_q]
    int32_t *d_K = nullptr;                   // [n_q][a_max][2]
    int32_t *d_bucket = nullptr;              // frequency lists by alias count
    long long *d_sk_wbegin = nullptr;
    int *d_sk_int = nullptr;

    ~Layout() {
        (void)hipSetDevice(key.device);
        (void)hipFree(d_pixbase);
        (void)hipFree(d_goff);
        (void)hipFree(d_tiles);
        (void)hipFree(d_prior);
        (void)hipFree(d_count);
        (void)hipFree(d_K);
        (void)hipFree(d_bucket);
        (void)hipFree(d_sk_wbegin);
        (void)hipFree(d_sk_int);
    }
};

// Builds a layout (host work plus blocking uploads on the device current).
dsp_status build_layout(const LayoutKey &key, const dsp_scan *scan, const dsp_optics *optics, const double *coords,
                        const double *weights, std::shared_ptr<Layout> &out) {
    const double t0 = now_ms();
    dsp_status st;
    auto L = std::make_shared<Layout>();
    L->key = key;
    if ((st = build_geometry(scan, optics, key.u, L->geo))) return st;
    Geometry &g = L->geo;
    const int max_nj = key.method == DSP_PHASE ? MAX_NJ_PHASE : MAX_NJ_COMPLEX;
    const int max_a = key.method == DSP_PHASE ? MAX_A_PHASE : MAX_A_SOLVE_COMPLEX;
    if (g.a_max > max_a) return fail(DSP_EALIAS, "alias count %d above the compiled maximum %d", g.a_max, max_a);
    if ((st = build_gram_tiles(g, max_nj, L->tg))) return st;
    if ((st = build_active(coords, weights, key.n_bf, optics, g.N, L->act))) return st;
    if (L->act.pix.empty()) return fail(DSP_EINVAL, "no bright-field pixel has a non-zero aperture weight");
    const int am = std::max(1, g.a_max);

    // prior per (frequency, alias)
    L->prior.assign((size_t)g.n_q * am, 1.0);
    const double sp = key.smooth;
    if (sp > 0.0) {
        for (int i = 0; i < g.n_q; ++i)
            for (int m = 0; m < g.count[i]; ++m) {
                const double qy = (double)g.K[((size_t)i * am + m) * 2] * g.dq;
                const double qx = (double)g.K[((size_t)i * am + m) * 2 + 1] * g.dq;
                const double b = 1.0 + (qy * qy + qx * qx) / (sp * sp);
                L->prior[(size_t)i * am + m] = b * b;
            }
    }
    // frequency lists by alias count
    L->bucket_off.assign(10, 0);
    L->bucket_n.assign(10, 0);
    for (int i = 0; i < g.n_q; ++i) L->bucket_n[g.count[i]]++;
    for (int A = 1; A <= 9; ++A) L->bucket_off[A] = L->bucket_off[A - 1] + L->bucket_n[A - 1];
    L->bucket.assign(g.n_q, 0);
    {
        std::vector<int> fill(L->bucket_off);
        for (int i = 0; i < g.n_q; ++i) L->bucket[fill[g.count[i]]++] = i;
    }

    // stream-K plan per tile group (one Gram launch per alias-slot count)
    const int n_groups = (int)L->tg.group_nj.size();
    const int n_pix = (int)L->act.pix.size();
    int n_cu = 0;
    HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, key.device));
    const ApertureDev apd = make_aperture_dev(optics);
    const double ra = std::sqrt(apd.rlim2);
    L->sk_waves.assign(n_groups, 0);
    L->wb_off.assign(n_groups, 0);
    L->so_off.assign(n_groups, 0);
    L->sf_off.assign(n_groups, 0);
    for (int gi = 0; gi < n_groups; ++gi) {
        const int nj = L->tg.group_nj[gi], nt = L->tg.group_n[gi];
        int bpc = 0;
        HIP_TRY(gram_occupancy(nj, key.method, &bpc));
        bpc = std::max(1, bpc);
        const long long total_it = (long long)nt * n_pix;
        const int W = (int)std::max(1LL, std::min((long long)bpc * n_cu * GRAM_ROUNDS, total_it / 64));
        std::vector<uint16_t> cost;
        gram_iteration_costs(L->tg.tiles.data() + L->tg.group_off[gi], nt, L->act.pix, g, ra, cost);
        StreamKPlan plan;
        plan_stream_k_iter(cost, nt, n_pix, W, plan);
        L->sk_waves[gi] = W;
        L->max_partial = std::max(L->max_partial, (size_t)plan.n_segs * gram_nacc(nj, key.method) * 64);
        L->wb_off[gi] = L->sk_wbegin.size();
        L->sk_wbegin.insert(L->sk_wbegin.end(), plan.wbegin.begin(), plan.wbegin.end());
        L->so_off[gi] = L->sk_int.size();
        L->sk_int.insert(L->sk_int.end(), plan.seg_off.begin(), plan.seg_off.end());
        L->sf_off[gi] = L->sk_int.size();
        L->sk_int.insert(L->sk_int.end(), plan.seg_first.begin(), plan.seg_first.end());
    }

    // device copies (blocking: a layout is built once and reused)
    if ((st = dev_alloc(&L->d_pixbase, L->act.pix.size())) || (st = dev_alloc(&L->d_goff, L->act.goff.size())) ||
        (st = dev_alloc(&L->d_tiles, L->tg.tiles.size())) ||
        (st = dev_alloc(&L->d_prior, L->prior.size())) || (st = dev_alloc(&L->d_count, g.count.size())) ||
        (st = dev_alloc(&L->d_K, g.K.size())) || (st = dev_alloc(&L->d_bucket, L->bucket.size())) ||
        (st = dev_alloc(&L->d_sk_wbegin, L->sk_wbegin.size())) || (st = dev_alloc(&L->d_sk_int, L->sk_int.size())))
        return st;
    HIP_TRY(hipMemcpy(L->d_pixbase, L->act.pix.data(), L->act.pix.size() * sizeof(PixelBase), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(L->d_goff, L->act.goff.data(), L->act.goff.size() * sizeof(long long), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(L->d_tiles, L->tg.tiles.data(), L->tg.tiles.size() * sizeof(GramTile), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(L->d_prior, L->prior.data(), L->prior.size() * sizeof(double), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(L->d_count, g.count.data(), g.count.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    if (!g.K.empty()) HIP_TRY(hipMemcpy(L->d_K, g.K.data(), g.K.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    if (!L->bucket.empty())
        HIP_TRY(hipMemcpy(L->d_bucket, L->bucket.data(), L->bucket.size() * sizeof(int32_t), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(L->d_sk_wbegin, L->sk_wbegin.data(), L->sk_wbegin.size() * sizeof(long long),
                      hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(L->d_sk_int, L->sk_int.data(), L->sk_int.size() * sizeof(int), hipMemcpyHostToDevice));
    L->host_ms = now_ms() - t0;
    out = L;
    return DSP_OK;
}

// Most recently used layouts (a handle keeps its own reference).  The
// caches are heap objects that are never destroyed: a layout's destructor
// frees device memory, and static destruction at process exit may run after
// the HIP runtime has shut down, so no HIP call may be left for it.
constexpr size_t LAYOUT_CACHE_SIZE = 4;
std::mutex g_layout_mu;
std::vector<std::shared_ptr<Layout>> &g_layouts = *new std::vector<std::shared_ptr<Layout>>();   // front = most recent

dsp_status get_layout(const LayoutKey &key, const dsp_scan *scan, const dsp_optics *optics, const double *coords,
                      const double *weights, std::shared_ptr<Layout> &out, bool &hit) {
    std::lock_guard<std::mutex> lock(g_layout_mu);
    for (size_t i = 0; i < g_layouts.size(); ++i) {
        if (g_layouts[i]->key == key) {
            out = g_layouts[i];
            g_layouts.erase(g_layouts.begin() + i);
            g_layouts.insert(g_layouts.begin(), out);
            hit = true;
            return DSP_OK;
        }
    }
    hit = false;
    dsp_status st = build_layout(key, scan, optics, coords, weights, out);
    if (st) return st;
    g_layouts.insert(g_layouts.begin(), out);
    if (g_layouts.size() > LAYOUT_CACHE_SIZE) g_layouts.pop_back();
    return DSP_OK;
}

// ---------------------------------------------------------------------------
// SSB layout, cached: active pixels, band tiles, stream-K plans per set count
// ---------------------------------------------------------------------------
struct SsbKey {
    int device = 0, n_scan = 0, soft = 0, n_bf = 0, has_band = 0;
    int up = 1;         // preview layouts: the upsampling u
    int preview = 0;    // 1: a preview layout (the key of its own cache)
    int noalloc = 0;    // host tables only, plans sized to the fixed scratch (dsp_ssb_noalloc)
    double step = 0, lam = 0, alpha = 0, dk = 0, lo = 0, hi = 0;
    std::vector<double> coords, weights;
    bool operator==(const SsbKey &o) const {
        return device == o.device && n_scan == o.n_scan && soft == o.soft && n_bf == o.n_bf && has_band == o.has_band &&
               up == o.up && preview == o.preview && noalloc == o.noalloc && step == o.step && lam == o.lam &&
               alpha == o.alpha && dk == o.dk && lo == o.lo && hi == o.hi && coords == o.coords &&
               weights == o.weights;
    }
};

struct SsbLayout {
    SsbKey key;
    ActiveSet act;
    std::vector<SsbTile> tiles;
    // per compiled set count (1, 2, 4, 8): waves, segments, stream-K tables
    int waves[4] = {0, 0, 0, 0};
    int n_segs[4] = {0, 0, 0, 0};
    std::vector<long long> wbegin[4];
    std::vector<int> seg_off[4], seg_first[4];
    PixelBase *d_pixbase = nullptr;
    long long *d_goff = nullptr;
    SsbTile *d_tiles = nullptr;
    long long *d_wbegin[4] = {nullptr, nullptr, nullptr, nullptr};
    int *d_seg_off[4] = {nullptr, nullptr, nullptr, nullptr};
    int *d_seg_first[4] = {nullptr, nullptr, nullptr, nullptr};
    size_t scratch_need[4] = {0, 0, 0, 0};   // noalloc: scratch bytes of a pass (0: does not fit)
    double host_ms = 0.0;
    ~SsbLayout() {
        // an allocation-free pass's layout holds no device memory: no HIP call
        if (key.noalloc) return;
        (void)hipSetDevice(key.device);
        (void)hipFree(d_pixbase);
        (void)hipFree(d_goff);
        (void)hipFree(d_tiles);
        for (int i = 0; i < 4; ++i) {
            (void)hipFree(d_wbegin[i]);
            (void)hipFree(d_seg_off[i]);
            (void)hipFree(d_seg_first[i]);
        }
    }
};

int maxb_index(int maxb) { return maxb == 1 ? 0 : (maxb == 2 ? 1 : (maxb == 4 ? 2 : 3)); }

// Scratch bytes of one allocation-free pass of up to maxb sets: the
// layout's device tables (trig table, pixels, plane offsets, tiles, stream-K
// tables), the per-call tables and the partial sums, each piece 256-byte
// aligned in the order ssb_impl carves them.
size_t noalloc_need(size_t n_pix, size_t n_tiles, int maxb, size_t W, size_t n_segs) {
    return carve_size(TRIG_N, sizeof(double2)) + carve_size(n_pix, sizeof(PixelBase)) +
           carve_size(n_pix, sizeof(long long)) + carve_size(n_tiles, sizeof(SsbTile)) +
           carve_size(W + 1, sizeof(long long)) + carve_size(W, sizeof(int)) + carve_size(n_tiles + 1, sizeof(int)) +
           carve_size(n_pix, sizeof(PixelRec)) + carve_size(n_segs * (size_t)ssb_nacc(maxb) * 64, sizeof(double)) +
           carve_size(n_tiles * (size_t)(maxb + 1), sizeof(double)) + carve_size(maxb + 1, sizeof(double)) +
           carve_size(std::max<size_t>(1, (size_t)maxb * n_pix * TAY_N), sizeof(double));
}

dsp_status build_ssb_layout(const SsbKey &key, const dsp_optics *optics, const double *coords,
                            const double *weights, std::shared_ptr<SsbLayout> &out) {
    const double t0 = now_ms();
    dsp_status st;
    auto L = std::make_shared<SsbLayout>();
    L->key = key;
    const int N = key.n_scan;
    const double dq = 1.0 / (N * key.step);
    if ((st = build_active(coords, weights, key.n_bf, optics, N, L->act))) return st;
    if (L->act.pix.empty()) return fail(DSP_EINVAL, "no bright-field pixel has a non-zero aperture weight");
    // lane groups over every stored entry inside the band (all of them
    // without one); the rest of the plane is zero
    const int nh = N / 2 + 1;
    auto keep = [&](int yh, int ix) {
        const double f = std::hypot((double)yh * dq, (double)ix * dq);
        return !key.has_band || (f >= key.lo && f <= key.hi);
    };
    for (const Lanes &grp : pack_line_runs(N, nh, -N / 2, (N - 1) / 2, nh, 16, keep)) {
        SsbTile t;
        std::memset(&t, 0, sizeof t);
        double sy = 0.0, sx = 0.0;
        for (size_t l = 0; l < grp.size(); ++l) {
            t.lyh[l] = grp[l].first;
            t.lix[l] = grp[l].second;
            t.valid |= 1ull << l;
            sy += grp[l].first;
            sx += grp[l].second;
        }
        t.cy = (float)(sy / grp.size());
        t.cx = (float)(sx / grp.size());
        // radius of the lanes about the stored centre, for the kernel's
        // per-pixel test (a bound: rounded up and widened by a part in 1e6)
        double rad = 0.0;
        for (size_t l = 0; l < grp.size(); ++l)
            rad = std::max(rad, std::hypot((double)t.lyh[l] - (double)t.cy, (double)t.lix[l] - (double)t.cx));
        t.rad = std::nextafter((float)(rad * (1.0 + 1e-6)), INFINITY);
        L->tiles.push_back(t);
    }
    const int n_tiles = (int)L->tiles.size();
    const int n_pix = (int)L->act.pix.size();
    const bool dev_tables = !key.noalloc;   // noalloc: the call copies the host tables into its scratch
    if (dev_tables) {
        if ((st = dev_alloc(&L->d_pixbase, (size_t)n_pix)) || (st = dev_alloc(&L->d_goff, (size_t)n_pix)) ||
            (st = dev_alloc(&L->d_tiles, (size_t)std::max(1, n_tiles))))
            return st;
        HIP_TRY(hipMemcpy(L->d_pixbase, L->act.pix.data(), sizeof(PixelBase) * n_pix, hipMemcpyHostToDevice));
        HIP_TRY(hipMemcpy(L->d_goff, L->act.goff.data(), sizeof(long long) * n_pix, hipMemcpyHostToDevice));
        if (n_tiles) HIP_TRY(hipMemcpy(L->d_tiles, L->tiles.data(), sizeof(SsbTile) * n_tiles, hipMemcpyHostToDevice));
    }
    if (n_tiles) {
        int n_cu = 0;
        HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, key.device));
        const double ra = std::sqrt(make_aperture_dev(optics).rlim2);
        // per (tile, pixel): the lobes the kernels' reach test admits; the
        // cost, in units of about four instructions, is a fixed part per
        // pixel (all the one-set kernel pays when no lobe is admitted), the
        // sets' sums, and per admitted lobe and set an evaluation
        std::vector<uint8_t> reach;
        ssb_reach_bits(L->tiles, L->act.pix, dq, ra, reach);
        static const int maxbs[4] = {1, 2, 4, 8};
        for (int mi = 0; mi < 4; ++mi) {
            const int maxb = maxbs[mi];
            struct Cost {
                const std::vector<uint8_t> *bits;
                int maxb;
                unsigned operator[](long long i) const {
                    const unsigned b = (*bits)[(size_t)i], nl = (b & 1u) + (b >> 1);
                    constexpr unsigned C_PIX = 14;   // G load and power; measured 6..14
                    if (maxb == 1 && nl == 0) return C_PIX;
                    return C_PIX + 2u * maxb + 20u * maxb * nl;
                }
            } cost{&reach, maxb};
            int bpc = 0;
            HIP_TRY(ssb_occupancy(maxb, &bpc));
            bpc = std::max(1, bpc);
            const long long total_it = (long long)n_tiles * n_pix;
            int W = (int)std::max(1LL, std::min((long long)bpc * n_cu * GRAM_ROUNDS, total_it / 64));
            if (key.noalloc) {
                // the most waves (down from the device path's count, halving)
                // whose tables and partial sums (at most W + n_tiles segments)
                // fit the fixed scratch; none: the pass does not fit
                while (W > 1 && noalloc_need(n_pix, n_tiles, maxb, W, (size_t)W + n_tiles) > NOALLOC_SCRATCH_BYTES)
                    W = std::max(1, W / 2);
                if (noalloc_need(n_pix, n_tiles, maxb, W, (size_t)W + n_tiles) > NOALLOC_SCRATCH_BYTES) {
                    L->scratch_need[mi] = 0;
                    L->waves[mi] = 0;
                    continue;
                }
            }
            StreamKPlan plan;
            plan_stream_k_iter(cost, n_tiles, n_pix, W, plan);
            L->waves[mi] = W;
            L->n_segs[mi] = plan.n_segs;
            L->wbegin[mi] = plan.wbegin;
            L->seg_off[mi] = plan.seg_off;
            L->seg_first[mi] = plan.seg_first;
            if (key.noalloc) {
                L->scratch_need[mi] = noalloc_need(n_pix, n_tiles, maxb, W, plan.n_segs);
                continue;
            }
            if ((st = dev_alloc(&L->d_wbegin[mi], plan.wbegin.size())) ||
                (st = dev_alloc(&L->d_seg_off[mi], plan.seg_off.size())) ||
                (st = dev_alloc(&L->d_seg_first[mi], plan.seg_first.size())))
                return st;
            HIP_TRY(hipMemcpy(L->d_wbegin[mi], plan.wbegin.data(), plan.wbegin.size() * sizeof(long long),
                              hipMemcpyHostToDevice));
            HIP_TRY(hipMemcpy(L->d_seg_off[mi], plan.seg_off.data(), plan.seg_off.size() * sizeof(int),
                              hipMemcpyHostToDevice));
            HIP_TRY(hipMemcpy(L->d_seg_first[mi], plan.seg_first.data(), plan.seg_first.size() * sizeof(int),
                              hipMemcpyHostToDevice));
        }
    }
    L->host_ms = now_ms() - t0;
    out = L;
    return DSP_OK;
}

// front = most recent (under g_layout_mu); never destroyed, like g_layouts
std::vector<std::shared_ptr<SsbLayout>> &g_ssb_layouts = *new std::vector<std::shared_ptr<SsbLayout>>();

// The allocation-free pass's layouts (host tables only) have a cache of
// their own: inserting one never evicts, and so never frees, a layout that
// holds device memory.
std::vector<std::shared_ptr<SsbLayout>> &g_ssb_noalloc_layouts = *new std::vector<std::shared_ptr<SsbLayout>>();

dsp_status get_ssb_layout(const SsbKey &key, const dsp_optics *optics, const double *coords, const double *weights,
                          std::shared_ptr<SsbLayout> &out) {
    std::lock_guard<std::mutex> lock(g_layout_mu);
    std::vector<std::shared_ptr<SsbLayout>> &cache = key.noalloc ? g_ssb_noalloc_layouts : g_ssb_layouts;
    for (size_t i = 0; i < cache.size(); ++i) {
        if (cache[i]->key == key) {
            out = cache[i];
            cache.erase(cache.begin() + i);
            cache.insert(cache.begin(), out);
            return DSP_OK;
        }
    }
    dsp_status st = build_ssb_layout(key, optics, coords, weights, out);
    if (st) return st;
    cache.insert(cache.begin(), out);
    if (cache.size() > LAYOUT_CACHE_SIZE) cache.pop_back();
    return DSP_OK;
}

// ---------------------------------------------------------------------------
// Preview layout, cached: the object fast path's corrected sum on the u-times
// finer grid ("Tilt-corrected SSB on CUDA: fit and preview speed", Changes:
// the 1x and 3x drag previews; "Where the 9 s of regularized preparation
// goes", Object-redraw fast path).  Fine frequency K reads G at K mod N, so
// every stored entry q feeds the fine K = q + j N: a lane holds one stored
// entry and its alias slots are those K (the Gram kernels' slot scheme with
// right sides only), so each G value is read once per pixel for all of its
// fine images.  A slot is written either directly (K in the fine half plane,
// Kx >= 0) or, where the half plane's K' = -K reads G through the Hermitian
// mirror (K'x mod N > N/2), as the conjugate at K'.
// ---------------------------------------------------------------------------
struct PreviewLayout {
    SsbKey key;
    ActiveSet act;
    TileGroups tg;
    std::vector<int> sk_waves;
    std::vector<size_t> wb_off, so_off, sf_off;
    std::vector<long long> sk_wbegin;
    std::vector<int> sk_int;
    size_t max_partial = 0;   // doubles of the largest group's partial sums
    PixelBase *d_pixbase = nullptr;
    long long *d_goff = nullptr;
    GramTile *d_tiles = nullptr;
    long long *d_sk_wbegin = nullptr;
    int *d_sk_int = nullptr;
    double host_ms = 0.0;
    ~PreviewLayout() {
        (void)hipSetDevice(key.device);
        (void)hipFree(d_pixbase);
        (void)hipFree(d_goff);
        (void)hipFree(d_tiles);
        (void)hipFree(d_sk_wbegin);
        (void)hipFree(d_sk_int);
    }
};

// The slots of stored entry (yh, ix): the offsets j whose fine K = (yh + jy N,
// ix + jx N) is within reach of two overlapping apertures (beyond it every
// lobe is exactly zero) and either lies in the computed part of the fine half
// plane itself (Kx >= 0; written at K) or has -K there with G read through
// the mirror, (-Kx) mod N > N/2 (written, conjugated, at -K).  The computed
// part: rows -(M/2)+1 .. (M-1)/2, columns 0 .. M/2-1, K != 0 (the Nyquist
// row and column stay zero; K = 0 is the uncorrected DC term).  Every
// computed fine K is the image of exactly one (entry, slot).
JSet preview_slots(int yh, int ix, int N, int u, double dq, double reach) {
    JSet js;
    const int M = u * N;
    auto computed = [M](int Ky, int Kx) {
        return Ky > -(M / 2) && Ky <= (M - 1) / 2 && Kx >= 0 && Kx < M / 2 && !(Ky == 0 && Kx == 0);
    };
    for (int jy = -u; jy <= u; ++jy) {
        const int Ky = yh + jy * N;
        for (int jx = -u; jx <= u; ++jx) {
            const int Kx = ix + jx * N;
            if (Kx >= 0 ? !computed(Ky, Kx) : (!computed(-Ky, -Kx) || (-Kx) % N <= N / 2)) continue;
            if (!(std::hypot((double)Ky * dq, (double)Kx * dq) < reach)) continue;
            js.emplace_back(jy, jx);
        }
    }
    return js;
}

void preview_finish_tile(GramTile &t, const JSet &js, const JSet (&lane_js)[64],
                         std::map<int, std::vector<std::pair<long long, GramTile>>> &by_nj) {
    t.nj = (int)js.size();
    for (int s = 0; s < t.nj; ++s) {
        t.jy[s] = (int8_t)js[s].first;
        t.jx[s] = (int8_t)js[s].second;
    }
    double sy = 0.0, sx = 0.0;
    int nv = 0;
    long long cost = 0;
    for (int l = 0; l < 64; ++l) {
        t.mask[l] = 0;
        if (t.qidx[l] < 0) continue;
        unsigned msk = 0;
        for (const auto &j : lane_js[l])
            msk |= 1u << (int)(std::lower_bound(js.begin(), js.end(), j) - js.begin());
        t.mask[l] = (uint16_t)msk;
        sy += t.lyh[l];
        sx += t.lix[l];
        ++nv;
        cost += (long long)lane_js[l].size();
    }
    t.cy = (float)(nv ? sy / nv : 0.0);
    t.cx = (float)(nv ? sx / nv : 0.0);
    double rad = 0.0;
    for (int l = 0; l < 64; ++l) {
        if (t.qidx[l] < 0) continue;
        rad = std::max(rad, std::hypot((double)t.lyh[l] - (double)t.cy, (double)t.lix[l] - (double)t.cx));
    }
    t.rad = std::nextafter((float)(rad * (1.0 + 1e-6)), INFINITY);
    by_nj[t.nj].emplace_back(-cost, t);
}

dsp_status build_preview_layout(const SsbKey &key, const dsp_optics *optics, const double *coords,
                                const double *weights, std::shared_ptr<PreviewLayout> &out) {
    const double t0 = now_ms();
    dsp_status st;
    auto L = std::make_shared<PreviewLayout>();
    L->key = key;
    const int N = key.n_scan, u = key.up, nh = N / 2 + 1;
    const double dq = 1.0 / (N * key.step);
    if ((st = build_active(coords, weights, key.n_bf, optics, N, L->act))) return st;
    if (L->act.pix.empty()) return fail(DSP_EINVAL, "no bright-field pixel has a non-zero aperture weight");
    const double reach = 2.0 * std::sqrt(make_aperture_dev(optics).rlim2) * (1.0 + 1e-9);

    // the stored entries (rows -N/2 .. N/2-1, columns 0 .. N/2) with at least
    // one slot; each entry's slots are worked out again where its tile is
    // built (cheap, and no per-entry storage at N = 8192)
    auto has = [&](int yh, int ix) { return !preview_slots(yh, ix, N, u, dq, reach).empty(); };

    // lane groups cut along G's lines; a group whose slot union exceeds
    // MAX_SLOTS splits into sub-tiles, greedily by lane, and a lane with more
    // slots than that alone spreads its slots over several sub-tiles
    std::map<int, std::vector<std::pair<long long, GramTile>>> by_nj;
    for (const Lanes &grp : pack_line_runs(N, nh, -N / 2, (N - 1) / 2, nh, 8, has)) {
        GramTile base;
        std::memset(&base, 0, sizeof base);
        JSet left[64];
        for (int l = 0; l < 64; ++l) {
            base.qidx[l] = -1;
            if (l >= (int)grp.size()) continue;
            base.lyh[l] = grp[l].first;
            base.lix[l] = grp[l].second;
            left[l] = preview_slots(grp[l].first, grp[l].second, N, u, dq, reach);
        }
        for (;;) {
            GramTile t = base;
            JSet js, lane_js[64];
            for (int l = 0; l < 64; ++l) {
                if (left[l].empty()) continue;
                JSet tryu = js;
                tryu.insert(tryu.end(), left[l].begin(), left[l].end());
                std::sort(tryu.begin(), tryu.end());
                tryu.erase(std::unique(tryu.begin(), tryu.end()), tryu.end());
                if ((int)tryu.size() <= MAX_SLOTS) {
                    js.swap(tryu);
                    lane_js[l].swap(left[l]);
                } else if (js.empty()) {
                    // one lane above the maximum: its first MAX_SLOTS slots
                    lane_js[l].assign(left[l].begin(), left[l].begin() + MAX_SLOTS);
                    left[l].erase(left[l].begin(), left[l].begin() + MAX_SLOTS);
                    js = lane_js[l];
                } else {
                    continue;
                }
                t.qidx[l] = 0;
            }
            if (js.empty()) break;
            preview_finish_tile(t, js, lane_js, by_nj);
        }
    }
    for (auto &kv : by_nj) {
        auto &v = kv.second;
        std::stable_sort(v.begin(), v.end(), [](const std::pair<long long, GramTile> &a,
                                                const std::pair<long long, GramTile> &b) { return a.first < b.first; });
        L->tg.group_nj.push_back(kv.first);
        L->tg.group_off.push_back((int)L->tg.tiles.size());
        L->tg.group_n.push_back((int)v.size());
        for (auto &p : v) L->tg.tiles.push_back(p.second);
    }

    // stream-K plan per group, as for the prepare's Gram launches
    const int n_groups = (int)L->tg.group_nj.size();
    const int n_pix = (int)L->act.pix.size();
    int n_cu = 0;
    HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, key.device));
    const double ra = std::sqrt(make_aperture_dev(optics).rlim2);
    Geometry g;
    g.N = N;
    g.u = u;
    g.dq = dq;
    L->sk_waves.assign(n_groups, 0);
    L->wb_off.assign(n_groups, 0);
    L->so_off.assign(n_groups, 0);
    L->sf_off.assign(n_groups, 0);
    for (int gi = 0; gi < n_groups; ++gi) {
        const int nj = L->tg.group_nj[gi], nt = L->tg.group_n[gi];
        int bpc = 0;
        HIP_TRY(gram_occupancy(nj, GRAM_PREVIEW, &bpc));
        bpc = std::max(1, bpc);
        const long long total_it = (long long)nt * n_pix;
        const int W = (int)std::max(1LL, std::min((long long)bpc * n_cu * GRAM_ROUNDS, total_it / 64));
        std::vector<uint16_t> cost;
        gram_iteration_costs(L->tg.tiles.data() + L->tg.group_off[gi], nt, L->act.pix, g, ra, cost);
        StreamKPlan plan;
        plan_stream_k_iter(cost, nt, n_pix, W, plan);
        L->sk_waves[gi] = W;
        L->max_partial = std::max(L->max_partial, (size_t)plan.n_segs * gram_nacc(nj, GRAM_PREVIEW) * 64);
        L->wb_off[gi] = L->sk_wbegin.size();
        L->sk_wbegin.insert(L->sk_wbegin.end(), plan.wbegin.begin(), plan.wbegin.end());
        L->so_off[gi] = L->sk_int.size();
        L->sk_int.insert(L->sk_int.end(), plan.seg_off.begin(), plan.seg_off.end());
        L->sf_off[gi] = L->sk_int.size();
        L->sk_int.insert(L->sk_int.end(), plan.seg_first.begin(), plan.seg_first.end());
    }
    if ((st = dev_alloc(&L->d_pixbase, (size_t)n_pix)) || (st = dev_alloc(&L->d_goff, (size_t)n_pix)) ||
        (st = dev_alloc(&L->d_tiles, std::max<size_t>(1, L->tg.tiles.size()))) ||
        (st = dev_alloc(&L->d_sk_wbegin, std::max<size_t>(1, L->sk_wbegin.size()))) ||
        (st = dev_alloc(&L->d_sk_int, std::max<size_t>(1, L->sk_int.size()))))
        return st;
    HIP_TRY(hipMemcpy(L->d_pixbase, L->act.pix.data(), sizeof(PixelBase) * n_pix, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(L->d_goff, L->act.goff.data(), sizeof(long long) * n_pix, hipMemcpyHostToDevice));
    if (!L->tg.tiles.empty())
        HIP_TRY(hipMemcpy(L->d_tiles, L->tg.tiles.data(), L->tg.tiles.size() * sizeof(GramTile),
                          hipMemcpyHostToDevice));
    if (!L->sk_wbegin.empty())
        HIP_TRY(hipMemcpy(L->d_sk_wbegin, L->sk_wbegin.data(), L->sk_wbegin.size() * sizeof(long long),
                          hipMemcpyHostToDevice));
    if (!L->sk_int.empty())
        HIP_TRY(hipMemcpy(L->d_sk_int, L->sk_int.data(), L->sk_int.size() * sizeof(int), hipMemcpyHostToDevice));
    L->host_ms = now_ms() - t0;
    out = L;
    return DSP_OK;
}

// front = most recent (under g_layout_mu); never destroyed, like g_layouts
std::vector<std::shared_ptr<PreviewLayout>> &g_preview_layouts = *new std::vector<std::shared_ptr<PreviewLayout>>();

dsp_status get_preview_layout(const SsbKey &key, const dsp_optics *optics, const double *coords,
                              const double *weights, std::shared_ptr<PreviewLayout> &out) {
    std::lock_guard<std::mutex> lock(g_layout_mu);
    for (size_t i = 0; i < g_preview_layouts.size(); ++i) {
        if (g_preview_layouts[i]->key == key) {
            out = g_preview_layouts[i];
            g_preview_layouts.erase(g_preview_layouts.begin() + i);
            g_preview_layouts.insert(g_preview_layouts.begin(), out);
            return DSP_OK;
        }
    }
    dsp_status st = build_preview_layout(key, optics, coords, weights, out);
    if (st) return st;
    g_preview_layouts.insert(g_preview_layouts.begin(), out);
    if (g_preview_layouts.size() > LAYOUT_CACHE_SIZE) g_preview_layouts.pop_back();
    return DSP_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// handle
// ---------------------------------------------------------------------------

struct dsp_handle {
    // references: the creator's, plus one per cache slot and per reference a
    // cache hands out; dsp_destroy drops one and frees at zero
    std::atomic<int> refs{1};
    int device = 0;
    int method = 0;
    std::shared_ptr<const Layout> L;
    int n_bf = 0;
    int D = 0, n_comp = 1;
    double host_ms = 0.0;
    bool layout_hit = false;
    // device, owned by the handle: pieces of one block from the device's
    // buffer cache (block, block_bytes)
    void *block = nullptr;
    size_t block_bytes = 0;
    // per stream the handle's buffers were used on, an event after the last
    // such work: the block goes back to the cache behind these events
    mutable std::vector<std::pair<hipStream_t, hipEvent_t>> uses;
    PixelRec *d_pix = nullptr;      // records with this optics' chi(k) and a(k)
    double *d_tay = nullptr;        // [n_pix][TAY_N] chi's Taylor coefficients about theta(k)
    double2 *d_sys = nullptr;       // [n_q][tri_size(D)]
    double *d_lam = nullptr;
    double2 *d_U = nullptr;
    double2 *d_c = nullptr;
    bool timing = false;
    bool count_work = false;
    bool slot_test = true;                    // DSP_FLAG_NO_SLOT_TEST clears it
    hipStream_t stream = nullptr;             // the prepare's stream
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    std::vector<int> gram_order;              // launch order of the tile groups
    std::vector<hipEvent_t> gram_ev;          // three per launch: start, Gram done, fixup done (timing)
    unsigned long long *d_work = nullptr;     // [tile][5] (DSP_FLAG_COUNT_WORK)

    // Records that work using the buffers has been queued on s.  Where no
    // event can be recorded, it waits for s here instead, so that the block
    // is free to reuse once the handle is destroyed.
    void mark(hipStream_t s) const {
        for (auto &u : uses) {
            if (u.first == s) {
                if (hipEventRecord(u.second, s) != hipSuccess) (void)hipStreamSynchronize(s);
                return;
            }
        }
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
            (void)hipStreamSynchronize(s);
            return;
        }
        if (hipEventRecord(e, s) != hipSuccess) {
            (void)hipEventDestroy(e);
            (void)hipStreamSynchronize(s);
            return;
        }
        uses.emplace_back(s, e);
    }

    // One block for the buffers: sizes in elements of PixelRec, double
    // (Taylor), double2 (systems), double (eigenvalues), double2 (U, c).
    dsp_status alloc(hipStream_t s, size_t n_pix, size_t n_tay, size_t n_sys, size_t n_lam, size_t n_U, size_t n_c) {
        const size_t total = carve_size(n_pix, sizeof(PixelRec)) + carve_size(n_tay, sizeof(double)) +
                             carve_size(n_sys, sizeof(double2)) + carve_size(n_lam, sizeof(double)) +
                             carve_size(n_U, sizeof(double2)) + carve_size(n_c, sizeof(double2));
        dsp_status st = pool_alloc(device, s, total, &block);
        if (st) return st;
        block_bytes = total;
        Carve cv{(char *)block};
        d_pix = n_pix ? cv.take<PixelRec>(n_pix) : nullptr;
        d_tay = n_tay ? cv.take<double>(n_tay) : nullptr;
        d_sys = n_sys ? cv.take<double2>(n_sys) : nullptr;
        d_lam = n_lam ? cv.take<double>(n_lam) : nullptr;
        d_U = n_U ? cv.take<double2>(n_U) : nullptr;
        d_c = n_c ? cv.take<double2>(n_c) : nullptr;
        return DSP_OK;
    }

    ~dsp_handle() {
        (void)hipSetDevice(device);
        std::vector<hipEvent_t> evs;
        for (auto &u : uses) evs.push_back(u.second);
        pool_release(device, block, block_bytes, std::move(evs));
        for (auto &e : ev)
            if (e) (void)hipEventDestroy(e);
        for (auto &e : gram_ev)
            if (e) (void)hipEventDestroy(e);
        (void)hipFree(d_work);
    }
};

// Marks a handle's use on a stream when the scope ends (success or failure).
struct MarkOnExit {
    const dsp_handle *h;
    hipStream_t s;
    ~MarkOnExit() {
        if (h) h->mark(s);
    }
};

// Phase eigenbasis of every frequency from the handle's systems, one Jacobi
// launch per alias count.
static dsp_status phase_eigen(dsp_handle *h, hipStream_t stream) {
    const Layout &L = *h->L;
    const Geometry &g = L.geo;
    const int am = std::max(1, g.a_max);
    EigParams ep;
    ep.sys = h->d_sys;
    ep.D = h->D;
    ep.a_max = am;
    ep.prior = L.d_prior;
    ep.lam = h->d_lam;
    ep.U = h->d_U;
    ep.c = h->d_c;
    // frequencies without aliases keep zero eigen data
    if (L.bucket_n[0] > 0) {
        HIP_TRY(launch_fill_zero(h->d_lam, (size_t)g.n_q * am, stream));
        HIP_TRY(launch_fill_zero((double *)h->d_U, (size_t)g.n_q * am * am * 2, stream));
        HIP_TRY(launch_fill_zero((double *)h->d_c, (size_t)g.n_q * am * 2, stream));
    }
    for (int A = 1; A <= 9; ++A) {
        if (L.bucket_n[A] == 0) continue;
        ep.qlist = L.d_bucket + L.bucket_off[A];
        ep.n = L.bucket_n[A];
        HIP_TRY(launch_eig(ep, A, stream));
    }
    return DSP_OK;
}

extern "C" {

const char *dsp_last_error(void) { return g_err.c_str(); }

void dsp_destroy(dsp_handle *h) {
    if (h && h->refs.fetch_sub(1, std::memory_order_acq_rel) == 1) delete h;
}

dsp_status dsp_geometry_counts(const dsp_scan *scan, const dsp_optics *optics, int upsampling, int *n_q, int *a_max,
                               int32_t *hist_out) {
    dsp_status st;
    if ((st = check_scan(scan)) || (st = check_optics(optics)) || (st = check_upsampling(upsampling))) return st;
    Geometry g;
    if ((st = build_geometry(scan, optics, upsampling, g))) return st;
    if (n_q) *n_q = g.n_q;
    if (a_max) *a_max = g.a_max;
    if (hist_out)
        for (int i = 0; i < 10; ++i) hist_out[i] = g.hist[i];
    return DSP_OK;
}

dsp_status dsp_alias_geometry(const dsp_scan *scan, const dsp_optics *optics, int upsampling, int32_t *q_host,
                              int32_t *count_host, int32_t *K_host) {
    dsp_status st;
    if ((st = check_scan(scan)) || (st = check_optics(optics)) || (st = check_upsampling(upsampling))) return st;
    Geometry g;
    if ((st = build_geometry(scan, optics, upsampling, g))) return st;
    if (q_host) std::memcpy(q_host, g.q.data(), g.q.size() * sizeof(int32_t));
    if (count_host) std::memcpy(count_host, g.count.data(), g.count.size() * sizeof(int32_t));
    if (K_host && g.a_max > 0) std::memcpy(K_host, g.K.data(), g.K.size() * sizeof(int32_t));
    return DSP_OK;
}

dsp_status dsp_active_bf(const double *bf_coords_host, int n_bf, const dsp_optics *optics, int32_t *idx_out,
                         int *n_active) {
    dsp_status st;
    if ((st = check_optics(optics))) return st;
    if (n_bf < 0 || (n_bf > 0 && !bf_coords_host)) return fail(DSP_EINVAL, "bad bf_coords");
    if (!n_active) return fail(DSP_EINVAL, "n_active is NULL");
    int n = 0;
    for (int i = 0; i < n_bf; ++i) {
        if (pixel_active(optics, bf_coords_host[2 * i], bf_coords_host[2 * i + 1])) {
            if (idx_out) idx_out[n] = i;
            ++n;
        }
    }
    *n_active = n;
    return DSP_OK;
}

dsp_status dsp_band_count(const dsp_scan *scan, const double *band_invA, int *count) {
    dsp_status st;
    if ((st = check_scan(scan))) return st;
    if (!count) return fail(DSP_EINVAL, "count is NULL");
    const int N = scan->n_scan;
    const double dq = 1.0 / (N * scan->step_A);
    int c = 0;
    for (int iy = 0; iy < N; ++iy) {
        const int yh = iy < N / 2 ? iy : iy - N;
        for (int ix = 0; ix <= N / 2; ++ix) {
            const double f = std::hypot((double)yh * dq, (double)ix * dq);
            if (!band_invA || (f >= band_invA[0] && f <= band_invA[1])) ++c;
        }
    }
    *count = c;
    return DSP_OK;
}

dsp_status dsp_chi_host(const dsp_optics *optics, const double *k_host, int n, double *chi_out) {
    dsp_status st;
    if ((st = check_optics(optics))) return st;
    if (n < 0 || (n > 0 && (!k_host || !chi_out))) return fail(DSP_EINVAL, "bad arguments");
    double c[CHI_NCOEF];
    chi_coefficients(optics, c);
    for (int i = 0; i < n; ++i) {
        const double ty = optics->wavelength_A * k_host[2 * i] + optics->tilt_rad[0];
        const double tx = optics->wavelength_A * k_host[2 * i + 1] + optics->tilt_rad[1];
        chi_out[i] = chi_poly(c, tx, ty);
    }
    return DSP_OK;
}

dsp_status dsp_chi_shift_host(const dsp_optics *optics, const double *k_host, const double *q_host, int n,
                              double *out) {
    dsp_status st;
    if ((st = check_optics(optics))) return st;
    if (n < 0 || (n > 0 && (!k_host || !q_host || !out))) return fail(DSP_EINVAL, "bad arguments");
    double c[CHI_NCOEF];
    chi_coefficients(optics, c);
    const double lam = optics->wavelength_A;
    for (int i = 0; i < n; ++i) {
        const double ty = lam * k_host[2 * i] + optics->tilt_rad[0];
        const double tx = lam * k_host[2 * i + 1] + optics->tilt_rad[1];
        double t[TAY_N], E, O;
        chi_taylor(c, tx, ty, t);
        chi_even_odd(t, c, lam * q_host[2 * i + 1], lam * q_host[2 * i], E, O);
        out[2 * i] = E - O;       // chi(k - Q) - chi(k)
        out[2 * i + 1] = E + O;   // chi(k + Q) - chi(k)
    }
    return DSP_OK;
}

dsp_status dsp_atan2_host(const double *y_host, const double *x_host, int n, double *out) {
    if (n < 0 || (n > 0 && (!y_host || !x_host || !out))) return fail(DSP_EINVAL, "bad arguments");
    double A[ATAN_N];
    atan_table_host(A);
    for (int i = 0; i < n; ++i) {
        const double x = x_host[i];
        out[i] = x == 0.0 ? std::atan2(y_host[i], x) : atan2_tab(y_host[i], x, 1.0 / x, A);
    }
    return DSP_OK;
}

dsp_status dsp_sincos_host(const double *x_host, int n, double *sin_out, double *cos_out) {
    if (n < 0 || (n > 0 && (!x_host || !sin_out || !cos_out))) return fail(DSP_EINVAL, "bad arguments");
    double2 T[TRIG_N];
    trig_table_host(T);
    for (int i = 0; i < n; ++i) sincos_tab(x_host[i], T, sin_out[i], cos_out[i]);
    return DSP_OK;
}

dsp_status dsp_prepare(const void *G_c64_dev, int n_bf, const double *bf_coords_host, const double *weights_host,
                       const dsp_scan *scan, const dsp_optics *optics, const dsp_prepare_opts *opts, void *hip_stream,
                       dsp_handle **out) {
    const double t0 = now_ms();
    dsp_status st;
    if (!out) return fail(DSP_EINVAL, "out is NULL");
    *out = nullptr;
    if ((st = check_scan(scan)) || (st = check_optics(optics))) return st;
    if (!opts) return fail(DSP_EINVAL, "opts is NULL");
    if ((st = check_upsampling(opts->upsampling))) return st;
    if (opts->method != DSP_PHASE && opts->method != DSP_COMPLEX) return fail(DSP_EINVAL, "unknown method %d", (int)opts->method);
    if (!G_c64_dev) return fail(DSP_EINVAL, "G is NULL");
    if (n_bf <= 0 || !bf_coords_host) return fail(DSP_EINVAL, "n_bf must be > 0 with bf_coords");
    if (!std::isfinite(opts->smoothness_invA)) return fail(DSP_EINVAL, "smoothness not finite");
    for (int i = 0; i < 2 * n_bf; ++i)
        if (!std::isfinite(bf_coords_host[i])) return fail(DSP_EINVAL, "bf_coords[%d] not finite", i / 2);
    if (weights_host)
        for (int i = 0; i < n_bf; ++i)
            if (!(weights_host[i] >= 0.0) || !std::isfinite(weights_host[i]))
                return fail(DSP_EINVAL, "weights[%d] must be finite and >= 0", i);
    if (opts->flags & ~(DSP_FLAG_TIMING | DSP_FLAG_COUNT_WORK | DSP_FLAG_NO_SLOT_TEST))
        return fail(DSP_EINVAL, "unknown flags 0x%x", (unsigned)opts->flags);
    hipStream_t stream = (hipStream_t)hip_stream;

    std::unique_ptr<dsp_handle> h(new dsp_handle());
    h->method = opts->method;
    h->n_bf = n_bf;
    h->timing = (opts->flags & DSP_FLAG_TIMING) != 0;
    h->count_work = (opts->flags & DSP_FLAG_COUNT_WORK) != 0;
    h->slot_test = (opts->flags & DSP_FLAG_NO_SLOT_TEST) == 0;
    h->stream = stream;
    HIP_TRY(hipGetDevice(&h->device));

    LayoutKey key;
    key.device = h->device;
    key.n_scan = scan->n_scan;
    key.step = scan->step_A;
    key.u = opts->upsampling;
    key.method = opts->method;
    key.soft = optics->soft_aperture;
    key.lam = optics->wavelength_A;
    key.alpha = optics->semiangle_rad;
    key.dk = optics->det_step_invA;
    key.smooth = opts->smoothness_invA > 0.0 ? opts->smoothness_invA : 0.0;
    key.n_bf = n_bf;
    key.coords.assign(bf_coords_host, bf_coords_host + 2 * (size_t)n_bf);
    if (weights_host) key.weights.assign(weights_host, weights_host + n_bf);
    std::shared_ptr<Layout> lay;
    if ((st = get_layout(key, scan, optics, bf_coords_host, weights_host, lay, h->layout_hit))) return st;
    h->L = lay;
    const Layout &L = *lay;
    const Geometry &g = L.geo;
    h->n_comp = h->method == DSP_PHASE ? 1 : 2;
    const int am = std::max(1, g.a_max);
    h->D = h->n_comp * am + 1;
    const int n_pix = (int)L.act.pix.size();

    // per-handle buffers: one block from the device's buffer cache; on every
    // way out of this call (the guard runs before h is freed on failure) an
    // event on the stream marks the last queued work with them
    const size_t n_sys = (size_t)g.n_q * tri_size(h->D);
    const bool ph = h->method == DSP_PHASE;
    if ((st = h->alloc(stream, (size_t)n_pix, (size_t)n_pix * TAY_N, n_sys, ph ? (size_t)g.n_q * am : 0,
                       ph ? (size_t)g.n_q * am * am : 0, ph ? (size_t)g.n_q * am : 0)))
        return st;
    MarkOnExit mark_guard{h.get(), stream};

    if (h->timing) {
        for (auto &e : h->ev) HIP_TRY(hipEventCreate(&e));
        HIP_TRY(hipEventRecord(h->ev[0], stream));
    }
    const ApertureDev apd = make_aperture_dev(optics);
    const OpticsDev opd = make_optics_dev(optics);
    HIP_TRY(launch_pixel_terms(L.d_pixbase, h->d_pix, n_pix, apd, opd, nullptr, 0, h->d_tay, stream));
    if (h->timing) HIP_TRY(hipEventRecord(h->ev[1], stream));

    GramParams gp;
    std::memset(&gp, 0, sizeof gp);
    gp.G = (const float2 *)G_c64_dev;
    gp.pix = h->d_pix;
    gp.tay = h->d_tay;
    gp.goff = L.d_goff;
    gp.n_pix = n_pix;
    gp.N = g.N;
    gp.nh = g.N / 2 + 1;
    gp.dq = g.dq;
    gp.ldq = optics->wavelength_A * g.dq;
    gp.ap = apd;
    gp.op = opd;
    gp.sys = h->d_sys;
    gp.a_max = am;
    gp.D = h->D;
    gp.slot_test = h->slot_test ? 1 : 0;
    if ((st = trig_table_device(h->device, &gp.trig))) return st;
    // partial sums live only for the Gram stage (the stream's scratch arena)
    double *d_partial = nullptr;
    {
        char *scr = nullptr;
        if ((st = arena_get(h->device, stream, std::max<size_t>(1, L.max_partial) * sizeof(double), &scr))) return st;
        d_partial = (double *)scr;
    }

    // largest groups first
    const int n_groups = (int)L.tg.group_nj.size();
    std::vector<int> order(n_groups);
    for (int i = 0; i < n_groups; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return L.tg.group_n[a] > L.tg.group_n[b]; });
    h->gram_order = order;
    if (h->timing) {
        h->gram_ev.assign(3 * order.size(), nullptr);
        for (auto &e : h->gram_ev) HIP_TRY(hipEventCreate(&e));
    }
    for (size_t oi = 0; oi < order.size(); ++oi) {
        const int gi = order[oi];
        gp.tiles = L.d_tiles + L.tg.group_off[gi];
        gp.wbegin = L.d_sk_wbegin + L.wb_off[gi];
        gp.seg_off = L.d_sk_int + L.so_off[gi];
        gp.seg_first = L.d_sk_int + L.sf_off[gi];
        gp.partial = d_partial;
        gp.n_waves = L.sk_waves[gi];
        if (h->timing) HIP_TRY(hipEventRecord(h->gram_ev[3 * oi], stream));
        HIP_TRY(launch_gram(gp, L.tg.group_nj[gi], h->method, gp.n_waves, stream));
        if (h->timing) HIP_TRY(hipEventRecord(h->gram_ev[3 * oi + 1], stream));
        HIP_TRY(launch_gram_fixup(gp, L.tg.group_nj[gi], h->method, L.tg.group_n[gi], stream));
        if (h->timing) HIP_TRY(hipEventRecord(h->gram_ev[3 * oi + 2], stream));
    }
    if (h->timing) HIP_TRY(hipEventRecord(h->ev[2], stream));

    if (h->method == DSP_PHASE && (st = phase_eigen(h.get(), stream))) return st;
    if (h->timing) HIP_TRY(hipEventRecord(h->ev[3], stream));
    if (h->count_work) {
        // instrumentation after the prepare's own kernels: work per tile
        if ((st = dev_alloc(&h->d_work, L.tg.tiles.size() * 5))) return st;
        for (int gi = 0; gi < n_groups; ++gi) {
            gp.tiles = L.d_tiles + L.tg.group_off[gi];
            HIP_TRY(launch_work_count(gp, h->method, L.tg.group_n[gi], h->d_work + (size_t)L.tg.group_off[gi] * 5,
                                      stream));
        }
    }
    h->host_ms = now_ms() - t0;
    *out = h.release();
    return DSP_OK;
}

dsp_status dsp_derive_phase(const dsp_handle *src, void *hip_stream, dsp_handle **out) {
    if (!out) return fail(DSP_EINVAL, "out is NULL");
    *out = nullptr;
    if (!src) return fail(DSP_EINVAL, "handle is NULL");
    if (src->method != DSP_COMPLEX) return fail(DSP_EINVAL, "the source handle must come from a complex prepare");
    const double t0 = now_ms();
    HIP_TRY(hipSetDevice(src->device));
    hipStream_t stream = (hipStream_t)hip_stream;
    dsp_status st;
    std::unique_ptr<dsp_handle> h(new dsp_handle());
    h->device = src->device;
    h->method = DSP_PHASE;
    h->L = src->L;
    h->n_bf = src->n_bf;
    h->n_comp = 1;
    h->layout_hit = true;
    h->stream = stream;
    const Geometry &g = h->L->geo;
    const int am = std::max(1, g.a_max);
    h->D = am + 1;
    if ((st = h->alloc(stream, 0, 0, (size_t)g.n_q * tri_size(h->D), (size_t)g.n_q * am, (size_t)g.n_q * am * am,
                       (size_t)g.n_q * am)))
        return st;
    MarkOnExit mark_guard{h.get(), stream};
    MarkOnExit mark_src{src, stream};   // the source's systems are read on this stream
    HIP_TRY(launch_phase_from_complex(src->d_sys, h->d_sys, am, g.n_q, stream));
    if ((st = phase_eigen(h.get(), stream))) return st;
    h->host_ms = now_ms() - t0;
    *out = h.release();
    return DSP_OK;
}

// ---------------------------------------------------------------------------
// two-slot prepared-model cache
// ---------------------------------------------------------------------------
}  // extern "C"

// Everything a prepared model depends on except its method, as doubles
// compared bit for bit (G by address and the caller's generation number).
static std::vector<double> cache_key(const void *G, unsigned long long g_version, int n_bf, const double *coords,
                                     const double *weights, const dsp_scan *scan, const dsp_optics *o,
                                     const dsp_prepare_opts *opts) {
    std::vector<double> k;
    auto put_u64 = [&](unsigned long long v) {
        double d;
        std::memcpy(&d, &v, sizeof d);
        k.push_back(d);
    };
    put_u64((unsigned long long)(uintptr_t)G);
    put_u64(g_version);
    k.push_back(n_bf);
    k.insert(k.end(), coords, coords + 2 * (size_t)n_bf);
    k.push_back(weights ? 1.0 : 0.0);
    if (weights) k.insert(k.end(), weights, weights + n_bf);
    k.push_back(scan->n_scan);
    k.push_back(scan->step_A);
    k.push_back(o->wavelength_A);
    k.push_back(o->semiangle_rad);
    k.push_back(o->det_step_invA);
    k.push_back(o->soft_aperture);
    k.push_back(o->tilt_rad[0]);
    k.push_back(o->tilt_rad[1]);
    k.push_back(o->depth_A);
    k.push_back(o->n_aber);
    for (int a = 0; a < o->n_aber && a < DSP_MAX_ABERRATIONS; ++a) {
        k.push_back(o->aber[a].n);
        k.push_back(o->aber[a].m);
        k.push_back(o->aber[a].c_A);
        k.push_back(o->aber[a].phi_rad);
    }
    k.push_back(opts->upsampling);
    k.push_back(opts->smoothness_invA);
    k.push_back(opts->flags);
    return k;
}

static bool same_key(const std::vector<double> &a, const std::vector<double> &b) {
    return a.size() == b.size() && (a.empty() || std::memcmp(a.data(), b.data(), a.size() * sizeof(double)) == 0);
}

struct dsp_cache {
    std::mutex mu;
    std::vector<double> key[2];   // per method
    dsp_handle *h[2] = {nullptr, nullptr};
    ~dsp_cache() {
        for (auto &x : h) dsp_destroy(x);
    }
};

extern "C" {

dsp_status dsp_cache_create(dsp_cache **out) {
    if (!out) return fail(DSP_EINVAL, "out is NULL");
    *out = new dsp_cache;
    return DSP_OK;
}

void dsp_cache_destroy(dsp_cache *c) { delete c; }

dsp_status dsp_cache_get(dsp_cache *c, const void *G_c64_dev, unsigned long long g_version, int n_bf,
                         const double *bf_coords_host, const double *weights_host, const dsp_scan *scan,
                         const dsp_optics *optics, const dsp_prepare_opts *opts, int derive, void *hip_stream,
                         dsp_handle **out, int *how) {
    if (!c || !out || !scan || !optics || !opts || !bf_coords_host || n_bf <= 0)
        return fail(DSP_EINVAL, "cache, out, scan, optics, opts and bf_coords must be given");
    if (opts->method != DSP_PHASE && opts->method != DSP_COMPLEX) return fail(DSP_EINVAL, "unknown method");
    *out = nullptr;
    const int m = opts->method == DSP_COMPLEX ? 1 : 0;
    std::vector<double> k = cache_key(G_c64_dev, g_version, n_bf, bf_coords_host, weights_host, scan, optics, opts);
    std::lock_guard<std::mutex> lock(c->mu);
    if (c->h[m] && same_key(c->key[m], k)) {
        c->h[m]->refs.fetch_add(1, std::memory_order_relaxed);   // the caller's reference
        *out = c->h[m];
        if (how) *how = 1;
        return DSP_OK;
    }
    dsp_handle *nh = nullptr;
    dsp_status st;
    int got = 0;
    if (m == 0 && derive && c->h[1] && same_key(c->key[1], k)) {
        st = dsp_derive_phase(c->h[1], hip_stream, &nh);
        got = 2;
    } else {
        st = dsp_prepare(G_c64_dev, n_bf, bf_coords_host, weights_host, scan, optics, opts, hip_stream, &nh);
    }
    if (st) return st;   // the slot keeps its model
    // the slot drops its reference to the old model; references handed out
    // earlier keep it alive until their holders release them
    dsp_destroy(c->h[m]);
    c->h[m] = nh;
    c->key[m] = std::move(k);
    nh->refs.fetch_add(1, std::memory_order_relaxed);   // the caller's reference
    *out = nh;
    if (how) *how = got;
    return DSP_OK;
}

dsp_status dsp_solve(dsp_handle *h, const double *strengths_host, int S, void *x_out_c128_dev, double *resid_out_dev,
                     void *hip_stream) {
    if (!h) return fail(DSP_EINVAL, "handle is NULL");
    if (S <= 0 || !strengths_host || !x_out_c128_dev) return fail(DSP_EINVAL, "need S > 0, strengths and x_out");
    const int per = h->method == DSP_PHASE ? 1 : 2;
    for (int i = 0; i < S * per; ++i)
        if (!(strengths_host[i] >= 0.0) || !std::isfinite(strengths_host[i]))
            return fail(DSP_EINVAL, "strength %d must be finite and >= 0", i);
    HIP_TRY(hipSetDevice(h->device));
    hipStream_t stream = (hipStream_t)hip_stream;
    MarkOnExit mark_guard{h, stream};
    const Geometry &g = h->L->geo;
    const int am = std::max(1, g.a_max);
    const int chunk = h->method == DSP_PHASE ? 64 : 32;
    double2 *x = (double2 *)x_out_c128_dev;
    for (int s0 = 0; s0 < S; s0 += chunk) {
        const int sn = std::min(chunk, S - s0);
        SolveParams sp;
        std::memset(&sp, 0, sizeof sp);
        sp.sys = h->d_sys;
        sp.D = h->D;
        sp.a_max = am;
        sp.n_q = g.n_q;
        sp.prior = h->L->d_prior;
        sp.lam = h->d_lam;
        sp.U = h->d_U;
        sp.c = h->d_c;
        for (int i = 0; i < sn * per; ++i) sp.strengths[i] = strengths_host[s0 * per + i];
        sp.S = sn;
        sp.scale = h->L->act.scale;
        sp.x = x + (size_t)s0 * h->n_comp * g.n_q * am;
        sp.resid = resid_out_dev ? resid_out_dev + (size_t)s0 * g.n_q : nullptr;
        for (int A = 0; A <= 9; ++A) {
            if (h->L->bucket_n[A] == 0) continue;
            sp.qlist = h->L->d_bucket + h->L->bucket_off[A];
            sp.n = h->L->bucket_n[A];
            HIP_TRY(launch_solve(sp, A, h->method, stream));
        }
    }
    return DSP_OK;
}

dsp_status dsp_scatter(const dsp_handle *h, const void *x_packed_c128_dev, int S, void *spec_out_c128_dev,
                       void *hip_stream) {
    if (!h) return fail(DSP_EINVAL, "handle is NULL");
    if (S <= 0 || !x_packed_c128_dev || !spec_out_c128_dev) return fail(DSP_EINVAL, "need S > 0, x and spec_out");
    HIP_TRY(hipSetDevice(h->device));
    hipStream_t stream = (hipStream_t)hip_stream;
    const Geometry &g = h->L->geo;
    const int nf = g.u * g.N;
    const size_t plane = (size_t)nf * (nf / 2 + 1);
    HIP_TRY(launch_fill_zero((double *)spec_out_c128_dev, (size_t)S * h->n_comp * plane * 2, stream));
    ScatterParams p;
    p.x = (const double2 *)x_packed_c128_dev;
    p.SC = S * h->n_comp;
    p.n_q = g.n_q;
    p.a_max = std::max(1, g.a_max);
    p.count = h->L->d_count;
    p.K = h->L->d_K;
    p.nf = nf;
    p.spec = (double2 *)spec_out_c128_dev;
    HIP_TRY(launch_scatter(p, stream));
    return DSP_OK;
}

dsp_status dsp_info(const dsp_handle *h, dsp_info_t *out) {
    if (!h || !out) return fail(DSP_EINVAL, "NULL argument");
    std::memset(out, 0, sizeof *out);
    const Geometry &g = h->L->geo;
    out->n_q = g.n_q;
    out->a_max = g.a_max;
    out->n_comp = h->n_comp;
    out->dim = h->D;
    out->n_bf = h->n_bf;
    out->n_active_bf = (int)h->L->act.pix.size();
    out->method = h->method;
    out->upsampling = g.u;
    out->n_scan = g.N;
    out->n_tiles = (int)h->L->tg.tiles.size();
    for (int i = 0; i < 10; ++i) out->alias_hist[i] = g.hist[i];
    out->scale = h->L->act.scale;
    out->g_bytes = (double)g.n_q * (double)h->L->act.pix.size() * 8.0;
    out->host_ms = h->host_ms;
    out->layout_ms = h->layout_hit ? 0.0 : h->L->host_ms;
    out->layout_cached = h->layout_hit ? 1 : 0;
    out->n_gram_launches = (int)std::min<size_t>(16, h->gram_order.size());
    for (int oi = 0; oi < out->n_gram_launches; ++oi) {
        const int gi = h->gram_order[oi];
        out->gram_nj[oi] = h->L->tg.group_nj[gi];
        out->gram_tiles[oi] = h->L->tg.group_n[gi];
        out->gram_waves[oi] = h->L->sk_waves[gi];
    }
    if ((h->timing && h->ev[3]) || (h->count_work && h->d_work)) HIP_TRY(hipSetDevice(h->device));
    // timings are filled once the prepare's last event has completed (no wait)
    bool timing_done = false;
    if (h->timing && h->ev[3]) {
        const hipError_t q = hipEventQuery(h->ev[3]);
        if (q != hipSuccess && q != hipErrorNotReady) HIP_TRY(q);
        timing_done = q == hipSuccess;
    }
    out->timing_ready = timing_done ? 1 : 0;
    if (timing_done) {
        float ms;
        HIP_TRY(hipEventElapsedTime(&ms, h->ev[0], h->ev[1]));
        out->stage_ms[0] = ms;
        HIP_TRY(hipEventElapsedTime(&ms, h->ev[1], h->ev[2]));
        out->stage_ms[1] = ms;
        HIP_TRY(hipEventElapsedTime(&ms, h->ev[2], h->ev[3]));
        out->stage_ms[2] = ms;
        HIP_TRY(hipEventElapsedTime(&ms, h->ev[0], h->ev[3]));
        out->stage_ms[3] = ms;
        for (int oi = 0; oi < out->n_gram_launches; ++oi) {
            HIP_TRY(hipEventElapsedTime(&ms, h->gram_ev[3 * oi], h->gram_ev[3 * oi + 1]));
            out->gram_ms[oi] = ms;
            HIP_TRY(hipEventElapsedTime(&ms, h->gram_ev[3 * oi + 1], h->gram_ev[3 * oi + 2]));
            out->gram_fixup_ms[oi] = ms;
        }
    }
    if (h->count_work && h->d_work) {
        // the counts are read with a blocking copy (instrumentation only)
        HIP_TRY(hipStreamSynchronize(h->stream));
        std::vector<unsigned long long> wk(h->L->tg.tiles.size() * 5, 0ull);
        HIP_TRY(hipMemcpy(wk.data(), h->d_work, wk.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
        double total = 0.0;
        for (size_t t = 0; t < h->L->tg.tiles.size(); ++t) total += (double)wk[t * 5 + 1];
        for (int oi = 0; oi < out->n_gram_launches; ++oi) {
            const int gi = h->gram_order[oi];
            for (int c = 0; c < 5; ++c) {
                double v = 0.0;
                for (int t = 0; t < h->L->tg.group_n[gi]; ++t) v += (double)wk[(size_t)(h->L->tg.group_off[gi] + t) * 5 + c];
                out->gram_work[oi][c] = v;
            }
        }
        out->lobes = total;
    }
    return DSP_OK;
}

dsp_status dsp_export_system(const dsp_handle *h, void *aug_out_c128_dev, double *eig_out_dev, void *hip_stream) {
    if (!h) return fail(DSP_EINVAL, "handle is NULL");
    HIP_TRY(hipSetDevice(h->device));
    hipStream_t stream = (hipStream_t)hip_stream;
    MarkOnExit mark_guard{h, stream};
    const Geometry &g = h->L->geo;
    if (aug_out_c128_dev) HIP_TRY(launch_export(h->d_sys, g.n_q, h->D, (double2 *)aug_out_c128_dev, stream));
    if (eig_out_dev) {
        if (h->method != DSP_PHASE) return fail(DSP_EINVAL, "eigenvalues exist for the phase method only");
        HIP_TRY(hipMemcpyAsync(eig_out_dev, h->d_lam, (size_t)g.n_q * std::max(1, g.a_max) * sizeof(double),
                               hipMemcpyDeviceToDevice, stream));
    }
    return DSP_OK;
}

dsp_status dsp_alias_table(const dsp_handle *h, int32_t *q_host, int32_t *count_host, int32_t *K_host) {
    if (!h) return fail(DSP_EINVAL, "handle is NULL");
    const Geometry &g = h->L->geo;
    if (q_host) std::memcpy(q_host, g.q.data(), g.q.size() * sizeof(int32_t));
    if (count_host) std::memcpy(count_host, g.count.data(), g.count.size() * sizeof(int32_t));
    if (K_host && g.a_max > 0) std::memcpy(K_host, g.K.data(), g.K.size() * sizeof(int32_t));
    return DSP_OK;
}

}  // extern "C"

// The SSB pass over complex64 G (GQ null) or herm16 G (GQ, gscale).
// Scratch of one SSB pass (the stream's arena, or the fixed scratch).
struct SsbPassBufs {
    PixelRec *pix;
    double *part;       // stream-K partial sums
    double *tile_part;  // [n_tiles][partial stride]
    double *tay;        // B tables [n_pix][TAY_N]
};

// Device copies of a pass's layout tables: the layout's own, or copies in
// the fixed scratch of the allocation-free pass.
struct SsbDevTables {
    const PixelBase *pixbase = nullptr;
    const long long *goff = nullptr;
    const SsbTile *tiles = nullptr;
    const long long *wbegin = nullptr;   // of the pass's compiled set count
    const int *seg_off = nullptr;
    const int *seg_first = nullptr;
    const double2 *trig = nullptr;
};

static dsp_status layout_tables(const SsbLayout &L, int mi, int device, SsbDevTables &t) {
    t.pixbase = L.d_pixbase;
    t.goff = L.d_goff;
    t.tiles = L.d_tiles;
    t.wbegin = L.d_wbegin[mi];
    t.seg_off = L.d_seg_off[mi];
    t.seg_first = L.d_seg_first[mi];
    return trig_table_device(device, &t.trig);
}

// One pass over G for B sets on layout L: pixel terms, then the SSB kernel
// with lanes on the stored (N, N/2 + 1) half plane writing S and N there.  The
// kernel takes both lobes' phases from each set's chi Taylor coefficients
// about theta(k) (bufs.tay: one evaluation of the even and odd parts in
// lambda q per pixel and set instead of the polynomial at both displaced
// points).
static dsp_status ssb_pass(const SsbLayout &L, const SsbDevTables &dt, const dsp_optics *sets_host, int B,
                           const void *G_c64_dev, const void *GQ_dev, const float *gscale_dev, int h16_rows, int N,
                           double2 *S_out, double *N_out, const SsbPassBufs &bufs, hipStream_t stream) {
    const int n_tiles = (int)L.tiles.size();
    const int n_pix = (int)L.act.pix.size();
    const int mi = maxb_index(ssb_maxb(B));
    const double dq = 1.0 / (N * L.key.step);
    const ApertureDev apd = make_aperture_dev(sets_host);
    SsbParams sp;
    std::memset(&sp, 0, sizeof sp);
    for (int b = 0; b < B; ++b) {
        const OpticsDev od = make_optics_dev(sets_host + b);
        // the pixel records once (set 0 writes them), the Taylor table per set
        // (the eight-set kernel computes its own: no tables)
        double *tb = ssb_maxb(B) >= 8 ? nullptr : bufs.tay + (size_t)b * n_pix * TAY_N;
        if (b == 0 || tb)
            HIP_TRY(launch_pixel_terms(dt.pixbase, b == 0 ? bufs.pix : nullptr, n_pix, apd, od, nullptr, 0, tb,
                                       stream));
        sp.tau_y[b] = od.tau_y;
        sp.tau_x[b] = od.tau_x;
        sp.pt2[b] = od.pt2;
        std::memcpy(sp.chi_c[b], od.chi_c, sizeof od.chi_c);
    }
    sp.G = (const float2 *)G_c64_dev;
    sp.GQ = (const short2 *)GQ_dev;
    sp.gscale = gscale_dev;
    sp.h16_rows = h16_rows;
    sp.plane = (long long)N * (N / 2 + 1);
    sp.pix = bufs.pix;
    sp.goff = dt.goff;
    sp.tay = bufs.tay;
    sp.n_pix = n_pix;
    sp.tiles = dt.tiles;
    sp.N = N;
    sp.nh = N / 2 + 1;
    sp.dq = dq;
    sp.ldq = sets_host[0].wavelength_A * dq;
    sp.B = B;
    sp.ap = apd;
    sp.lam = sets_host[0].wavelength_A;
    sp.S_out = S_out;
    sp.N_out = N_out;
    sp.wbegin = dt.wbegin;
    sp.seg_off = dt.seg_off;
    sp.seg_first = dt.seg_first;
    sp.partial = bufs.part;
    sp.trig = dt.trig;
    HIP_TRY(launch_ssb(sp, L.waves[mi], n_tiles, bufs.tile_part, stream));
    return DSP_OK;
}

// Inverse real FFTs (hipFFT Z2D, unnormalized): batch planes of (m, m/2 + 1)
// complex -> (m, m) real.  Plans are made once per (device, m, batch) and
// kept for the process (their work areas with them); a plan is bound to the
// caller's stream for each execution under the lock.  hipFFT may overwrite
// the input.
static std::mutex g_fft_mu;
static std::map<std::tuple<int, int, int>, hipfftHandle> g_fft_plans;

static dsp_status fft_z2d(int device, int m, int batch, double2 *in, double *out, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_fft_mu);
    const auto key = std::make_tuple(device, m, batch);
    hipfftHandle plan;
    auto it = g_fft_plans.find(key);
    if (it == g_fft_plans.end()) {
        hipfftResult r;
        if (batch == 1) {
            r = hipfftPlan2d(&plan, m, m, HIPFFT_Z2D);
        } else {
            int n[2] = {m, m};
            r = hipfftPlanMany(&plan, 2, n, nullptr, 1, m * (m / 2 + 1), nullptr, 1, m * m, HIPFFT_Z2D, batch);
        }
        if (r != HIPFFT_SUCCESS) return fail(DSP_EDEVICE, "hipfft plan %d x %d (batch %d): error %d", m, m, batch, (int)r);
        g_fft_plans[key] = plan;
    } else {
        plan = it->second;
    }
    hipfftResult r = hipfftSetStream(plan, stream);
    if (r == HIPFFT_SUCCESS) r = hipfftExecZ2D(plan, (hipfftDoubleComplex *)in, (hipfftDoubleReal *)out);
    if (r != HIPFFT_SUCCESS) return fail(DSP_EDEVICE, "hipfft Z2D %d x %d (batch %d): error %d", m, m, batch, (int)r);
    return DSP_OK;
}

// Validation shared by the passes over G.
static dsp_status check_pass_args(const dsp_scan *scan, const dsp_optics *optics, int n_bf, const double *coords,
                                  const double *weights) {
    dsp_status st;
    if ((st = check_scan(scan)) || (st = check_optics(optics))) return st;
    if (n_bf <= 0 || !coords) return fail(DSP_EINVAL, "n_bf must be > 0 with bf_coords");
    for (int i = 0; i < 2 * n_bf; ++i)
        if (!std::isfinite(coords[i])) return fail(DSP_EINVAL, "bf_coords[%d] not finite", i / 2);
    if (weights)
        for (int i = 0; i < n_bf; ++i)
            if (!(weights[i] >= 0.0) || !std::isfinite(weights[i]))
                return fail(DSP_EINVAL, "weights[%d] must be finite and >= 0", i);
    return DSP_OK;
}

static SsbKey pass_key(int device, const dsp_scan *scan, const dsp_optics *o, int n_bf, const double *coords,
                       const double *weights) {
    SsbKey key;
    key.device = device;
    key.n_scan = scan->n_scan;
    key.step = scan->step_A;
    key.soft = o->soft_aperture;
    key.lam = o->wavelength_A;
    key.alpha = o->semiangle_rad;
    key.dk = o->det_step_invA;
    key.n_bf = n_bf;
    key.coords.assign(coords, coords + 2 * (size_t)n_bf);
    if (weights) key.weights.assign(weights, weights + n_bf);
    return key;
}

// noalloc: every device buffer of the pass, layout tables included, comes
// from the fixed scratch (no device allocation); the plan is the one sized
// to it.
static dsp_status ssb_impl(const void *G_c64_dev, const void *GQ_dev, const float *gscale_dev, int h16_rows, int n_bf,
                           const double *bf_coords_host, const double *weights_host, const dsp_scan *scan,
                           const dsp_optics *sets_host, int B, const double *band_invA, void *S_out_c128_dev,
                           double *norm_out_dev, double *agreement_out_host, void *hip_stream, bool noalloc = false) {
    dsp_status st;
    if ((st = check_scan(scan))) return st;
    if (!sets_host || B < 1 || B > MAX_SETS) return fail(DSP_EINVAL, "need 1 <= B <= %d optics sets", MAX_SETS);
    for (int b = 0; b < B; ++b)
        if ((st = check_optics(sets_host + b))) return st;
    for (int b = 1; b < B; ++b) {
        const dsp_optics &a = sets_host[0], &c = sets_host[b];
        if (a.wavelength_A != c.wavelength_A || a.semiangle_rad != c.semiangle_rad ||
            a.det_step_invA != c.det_step_invA || a.soft_aperture != c.soft_aperture)
            return fail(DSP_EINVAL, "set %d: aperture parameters differ from set 0", b);
    }
    if (!G_c64_dev && !(GQ_dev && gscale_dev)) return fail(DSP_EINVAL, "G is NULL");
    if (n_bf <= 0 || !bf_coords_host) return fail(DSP_EINVAL, "n_bf must be > 0 with bf_coords");
    if (band_invA && !(band_invA[0] <= band_invA[1])) return fail(DSP_EINVAL, "band must satisfy lo <= hi");
    for (int i = 0; i < 2 * n_bf; ++i)
        if (!std::isfinite(bf_coords_host[i])) return fail(DSP_EINVAL, "bf_coords[%d] not finite", i / 2);
    if (weights_host)
        for (int i = 0; i < n_bf; ++i)
            if (!(weights_host[i] >= 0.0) || !std::isfinite(weights_host[i]))
                return fail(DSP_EINVAL, "weights[%d] must be finite and >= 0", i);
    hipStream_t stream = (hipStream_t)hip_stream;
    const int N = scan->n_scan, nh = N / 2 + 1;
    const double dq = 1.0 / (N * scan->step_A);
    int device = 0;
    HIP_TRY(hipGetDevice(&device));

    SsbKey key;
    key.device = device;
    key.n_scan = N;
    key.step = scan->step_A;
    key.soft = sets_host[0].soft_aperture;
    key.lam = sets_host[0].wavelength_A;
    key.alpha = sets_host[0].semiangle_rad;
    key.dk = sets_host[0].det_step_invA;
    key.has_band = band_invA ? 1 : 0;
    key.lo = band_invA ? band_invA[0] : 0.0;
    key.hi = band_invA ? band_invA[1] : 0.0;
    key.n_bf = n_bf;
    key.noalloc = noalloc ? 1 : 0;
    key.coords.assign(bf_coords_host, bf_coords_host + 2 * (size_t)n_bf);
    if (weights_host) key.weights.assign(weights_host, weights_host + n_bf);
    std::shared_ptr<SsbLayout> lay;
    if ((st = get_ssb_layout(key, sets_host, bf_coords_host, weights_host, lay))) return st;
    const SsbLayout &L = *lay;
    const int n_tiles = (int)L.tiles.size();
    const int n_pix = (int)L.act.pix.size();
    const int maxb = ssb_maxb(B);
    const int mi = maxb_index(maxb);
    const int stride = ssb_partial_stride(B);
    const size_t plane = (size_t)N * nh;
    if (noalloc && n_tiles > 0 && L.waves[mi] == 0)
        return fail(DSP_ENOMEM,
                    "the allocation-free SSB pass of %d sets over %d pixels and %d frequency tiles needs more than "
                    "its fixed %zu-byte scratch",
                    B, n_pix, n_tiles, NOALLOC_SCRATCH_BYTES);
    if (S_out_c128_dev && band_invA) HIP_TRY(launch_fill_zero((double *)S_out_c128_dev, (size_t)B * plane * 2, stream));
    if (norm_out_dev && band_invA) HIP_TRY(launch_fill_zero(norm_out_dev, (size_t)B * plane, stream));
    if (n_tiles == 0) {
        if (agreement_out_host) {
            HIP_TRY(hipStreamSynchronize(stream));
            for (int b = 0; b < B; ++b) agreement_out_host[b] = 0.0;
        }
        return DSP_OK;
    }

    // per-call tables: the stream's scratch arena, or (noalloc) the fixed
    // scratch, which also takes copies of the layout's tables
    const size_t n_part = (size_t)L.n_segs[mi] * ssb_nacc(maxb) * 64;
    const size_t n_tay = (size_t)B * n_pix * TAY_N;
    SsbDevTables dt;
    char *scr = nullptr;
    if (noalloc) {
        HIP_TRY(noalloc_scratch(&scr));
        // every piece must lie inside the scratch: the plan was sized to it
        // (noalloc_need carves the same pieces in the same order)
        const size_t total = noalloc_need(n_pix, n_tiles, maxb, L.waves[mi], L.n_segs[mi]);
        if (total != L.scratch_need[mi] || total > NOALLOC_SCRATCH_BYTES)
            return fail(DSP_ENOMEM, "allocation-free SSB pass: %zu bytes of scratch planned, %zu held", total,
                        NOALLOC_SCRATCH_BYTES);
        Carve tv{scr};
        double2 *d_trig = tv.take<double2>(TRIG_N);
        PixelBase *d_pb = tv.take<PixelBase>(n_pix);
        long long *d_go = tv.take<long long>(n_pix);
        SsbTile *d_ti = tv.take<SsbTile>(n_tiles);
        long long *d_wb = tv.take<long long>(L.wbegin[mi].size());
        int *d_so = tv.take<int>(L.seg_off[mi].size());
        int *d_sf = tv.take<int>(L.seg_first[mi].size());
        static const std::vector<double2> trig_host = [] {
            std::vector<double2> t(TRIG_N);
            trig_table_host(t.data());
            return t;
        }();
        // pageable host sources: each copy has consumed its source when the call returns
        HIP_TRY(hipMemcpyAsync(d_trig, trig_host.data(), TRIG_N * sizeof(double2), hipMemcpyHostToDevice, stream));
        HIP_TRY(hipMemcpyAsync(d_pb, L.act.pix.data(), n_pix * sizeof(PixelBase), hipMemcpyHostToDevice, stream));
        HIP_TRY(hipMemcpyAsync(d_go, L.act.goff.data(), n_pix * sizeof(long long), hipMemcpyHostToDevice, stream));
        HIP_TRY(hipMemcpyAsync(d_ti, L.tiles.data(), n_tiles * sizeof(SsbTile), hipMemcpyHostToDevice, stream));
        HIP_TRY(hipMemcpyAsync(d_wb, L.wbegin[mi].data(), L.wbegin[mi].size() * sizeof(long long),
                               hipMemcpyHostToDevice, stream));
        HIP_TRY(hipMemcpyAsync(d_so, L.seg_off[mi].data(), L.seg_off[mi].size() * sizeof(int), hipMemcpyHostToDevice,
                               stream));
        HIP_TRY(hipMemcpyAsync(d_sf, L.seg_first[mi].data(), L.seg_first[mi].size() * sizeof(int),
                               hipMemcpyHostToDevice, stream));
        dt.trig = d_trig;
        dt.pixbase = d_pb;
        dt.goff = d_go;
        dt.tiles = d_ti;
        dt.wbegin = d_wb;
        dt.seg_off = d_so;
        dt.seg_first = d_sf;
        scr += tv.off;
    } else {
        const size_t need = carve_size(n_pix, sizeof(PixelRec)) + carve_size(n_part, sizeof(double)) +
                            carve_size((size_t)n_tiles * stride, sizeof(double)) + carve_size(B + 1, sizeof(double)) +
                            carve_size(std::max<size_t>(1, n_tay), sizeof(double));
        if ((st = arena_get(device, stream, need, &scr))) return st;
        if ((st = layout_tables(L, mi, device, dt))) return st;
    }
    Carve cv{scr};
    PixelRec *d_pix = cv.take<PixelRec>(n_pix);
    double *d_part = cv.take<double>(n_part);
    double *d_tile_part = cv.take<double>((size_t)n_tiles * stride);
    double *d_E = cv.take<double>(B + 1);
    double *d_tay = cv.take<double>(std::max<size_t>(1, n_tay));

    SsbPassBufs bufs{d_pix, d_part, d_tile_part, d_tay};
    if ((st = ssb_pass(L, dt, sets_host, B, G_c64_dev, GQ_dev, gscale_dev, h16_rows, N, (double2 *)S_out_c128_dev,
                       norm_out_dev, bufs, stream)))
        return st;
    std::vector<double> E(B + 1, 0.0);
    if (agreement_out_host) {
        HIP_TRY(launch_agreement(d_tile_part, n_tiles, B, d_E, stream));
        HIP_TRY(hipMemcpyAsync(E.data(), d_E, sizeof(double) * (B + 1), hipMemcpyDeviceToHost, stream));
    }
    if (agreement_out_host) {
        HIP_TRY(hipStreamSynchronize(stream));
        for (int b = 0; b < B; ++b) agreement_out_host[b] = E[b];
    }
    return DSP_OK;
}

extern "C" {

dsp_status dsp_ssb(const void *G_c64_dev, int n_bf, const double *bf_coords_host, const double *weights_host,
                   const dsp_scan *scan, const dsp_optics *sets_host, int B, const double *band_invA,
                   void *S_out_c128_dev, double *norm_out_dev, double *agreement_out_host, void *hip_stream) {
    if (!G_c64_dev) return fail(DSP_EINVAL, "G is NULL");
    return ssb_impl(G_c64_dev, nullptr, nullptr, 0, n_bf, bf_coords_host, weights_host, scan, sets_host, B, band_invA,
                    S_out_c128_dev, norm_out_dev, agreement_out_host, hip_stream);
}

dsp_status dsp_ssb_noalloc(const void *G_c64_dev, int n_bf, const double *bf_coords_host, const double *weights_host,
                           const dsp_scan *scan, const dsp_optics *sets_host, int B, const double *band_invA,
                           void *S_out_c128_dev, double *norm_out_dev, double *agreement_out_host, void *hip_stream) {
    if (!G_c64_dev) return fail(DSP_EINVAL, "G is NULL");
    return ssb_impl(G_c64_dev, nullptr, nullptr, 0, n_bf, bf_coords_host, weights_host, scan, sets_host, B, band_invA,
                    S_out_c128_dev, norm_out_dev, agreement_out_host, hip_stream, true);
}

dsp_status dsp_ssb_herm16(const void *Q_i16_dev, const float *scale_dev, int row_scales, int n_bf,
                          const double *bf_coords_host, const double *weights_host, const dsp_scan *scan,
                          const dsp_optics *sets_host, int B, const double *band_invA, void *S_out_c128_dev,
                          double *norm_out_dev, double *agreement_out_host, void *hip_stream) {
    if (!Q_i16_dev || !scale_dev) return fail(DSP_EINVAL, "Q and scale must be non-NULL");
    return ssb_impl(nullptr, Q_i16_dev, scale_dev, row_scales ? 1 : 0, n_bf, bf_coords_host, weights_host, scan,
                    sets_host, B, band_invA, S_out_c128_dev, norm_out_dev, agreement_out_host, hip_stream);
}

dsp_status dsp_preview(const void *G_c64_dev, int n_bf, const double *bf_coords_host, const double *weights_host,
                       const dsp_scan *scan, const dsp_optics *optics, int upsampling, void *spec_out_c128_dev,
                       double *phase_out_dev, void *hip_stream) {
    dsp_status st;
    if ((st = check_pass_args(scan, optics, n_bf, bf_coords_host, weights_host))) return st;
    if (!G_c64_dev) return fail(DSP_EINVAL, "G is NULL");
    if (upsampling < 1 || upsampling > 4) return fail(DSP_EUNSUPPORTED, "upsampling %d not in 1..4", upsampling);
    if (!spec_out_c128_dev && !phase_out_dev) return fail(DSP_EINVAL, "no output requested");
    hipStream_t stream = (hipStream_t)hip_stream;
    const int N = scan->n_scan, M = upsampling * N, mh = M / 2 + 1;
    const long long n_half = (long long)M * mh;
    int device = 0;
    HIP_TRY(hipGetDevice(&device));
    SsbKey key = pass_key(device, scan, optics, n_bf, bf_coords_host, weights_host);
    key.up = upsampling;
    key.preview = 1;
    std::shared_ptr<PreviewLayout> lay;
    if ((st = get_preview_layout(key, optics, bf_coords_host, weights_host, lay))) return st;
    const PreviewLayout &L = *lay;
    const int n_pix = (int)L.act.pix.size();
    const size_t need = carve_size(n_pix, sizeof(PixelRec)) + carve_size(std::max<size_t>(1, L.max_partial), sizeof(double)) +
                        carve_size((size_t)n_half, sizeof(double2)) + carve_size(1, sizeof(double2));
    char *scr = nullptr;
    if ((st = arena_get(device, stream, need, &scr))) return st;
    Carve cv{scr};
    PixelRec *d_pix = cv.take<PixelRec>(n_pix);
    double *d_partial = cv.take<double>(std::max<size_t>(1, L.max_partial));
    double2 *d_S = cv.take<double2>((size_t)n_half);
    double2 *d_dc = cv.take<double2>(1);
    // S on the fine half plane (zero where no slot writes: K = 0, the Nyquist
    // lines and beyond reach)
    HIP_TRY(launch_fill_zero((double *)d_S, (size_t)n_half * 2, stream));
    const ApertureDev apd = make_aperture_dev(optics);
    const OpticsDev opd = make_optics_dev(optics);
    HIP_TRY(launch_pixel_terms(L.d_pixbase, d_pix, n_pix, apd, opd, nullptr, 0, nullptr, stream));
    GramParams gp;
    std::memset(&gp, 0, sizeof gp);
    gp.G = (const float2 *)G_c64_dev;
    gp.pix = d_pix;
    gp.goff = L.d_goff;
    gp.n_pix = n_pix;
    gp.N = N;
    gp.nh = N / 2 + 1;
    gp.dq = 1.0 / (N * scan->step_A);
    gp.ldq = optics->wavelength_A * gp.dq;
    gp.ap = apd;
    gp.op = opd;
    gp.sys = d_S;
    gp.slot_test = 1;
    gp.fine_M = M;
    gp.fine_mh = mh;
    gp.partial = d_partial;
    if ((st = trig_table_device(device, &gp.trig))) return st;
    for (size_t gi = 0; gi < L.tg.group_nj.size(); ++gi) {
        gp.tiles = L.d_tiles + L.tg.group_off[gi];
        gp.wbegin = L.d_sk_wbegin + L.wb_off[gi];
        gp.seg_off = L.d_sk_int + L.so_off[gi];
        gp.seg_first = L.d_sk_int + L.sf_off[gi];
        gp.n_waves = L.sk_waves[gi];
        HIP_TRY(launch_gram(gp, L.tg.group_nj[gi], GRAM_PREVIEW, gp.n_waves, stream));
        HIP_TRY(launch_gram_fixup(gp, L.tg.group_nj[gi], GRAM_PREVIEW, L.tg.group_n[gi], stream));
    }
    HIP_TRY(launch_preview_dc(L.d_pixbase, L.d_goff, n_pix, (const float2 *)G_c64_dev, d_dc, stream));
    if (spec_out_c128_dev) HIP_TRY(launch_preview_spectrum(d_S, d_dc, n_half, (double2 *)spec_out_c128_dev, stream));
    if (phase_out_dev) {
        if ((st = fft_z2d(device, M, 1, d_S, phase_out_dev, stream))) return st;
        HIP_TRY(launch_preview_phase(phase_out_dev, (long long)M * M, d_dc, stream));
    }
    return DSP_OK;
}

dsp_status dsp_loss(const void *G_c64_dev, int n_bf, const double *bf_coords_host, const double *weights_host,
                    const dsp_scan *scan, const dsp_optics *optics, double *mean_phase_out_dev, double *loss_out_host,
                    void *hip_stream) {
    dsp_status st;
    if ((st = check_pass_args(scan, optics, n_bf, bf_coords_host, weights_host))) return st;
    if (!G_c64_dev) return fail(DSP_EINVAL, "G is NULL");
    if (!mean_phase_out_dev && !loss_out_host) return fail(DSP_EINVAL, "no output requested");
    hipStream_t stream = (hipStream_t)hip_stream;
    const int N = scan->n_scan, nh = N / 2 + 1;
    const long long plane = (long long)N * nh, nn = (long long)N * N;
    int device = 0;
    HIP_TRY(hipGetDevice(&device));
    std::shared_ptr<SsbLayout> lay;
    if ((st = get_ssb_layout(pass_key(device, scan, optics, n_bf, bf_coords_host, weights_host), optics,
                             bf_coords_host, weights_host, lay)))
        return st;
    const SsbLayout &L = *lay;
    const int n_pix = (int)L.act.pix.size();
    double W = 0.0;
    for (const PixelBase &p : L.act.pix) W += p.w;
    if (!(W > 0.0)) return fail(DSP_EINVAL, "the active pixels' weights sum to zero");
    // power-of-two N up to 1024: the fused transforms (the column pass
    // computes the corrected values, the row pass the phase moments); else
    // the corrected planes, hipFFT's inverse real transform and the moments
    const bool fused = N >= 8 && N <= 1024 && (N & (N - 1)) == 0;
    // chunk of pixels per batch: about 1 GB of planes (and real images)
    const size_t per_pix = (size_t)plane * sizeof(double2) + (fused ? 0 : (size_t)nn * sizeof(double));
    const int CH = (int)std::max<size_t>(1, std::min<size_t>(256, ((size_t)1 << 30) / per_pix));
    // fused: pixel groups of the row pass (about 4096 blocks of rows), each
    // with partial moment planes
    const int NG = fused ? std::max(1, std::min(CH, 4096 / (N / 2))) : 0;
    const int nb = loss_blocks(nn);
    const size_t need = carve_size(n_pix, sizeof(PixelRec)) + carve_size((size_t)CH * plane, sizeof(double2)) +
                        carve_size(fused ? 1 : (size_t)CH * nn, sizeof(double)) + carve_size(CH, sizeof(double2)) +
                        2 * carve_size((size_t)nn, sizeof(double)) + carve_size(nb, sizeof(double)) +
                        carve_size(1, sizeof(double)) + 2 * carve_size(std::max<size_t>(1, (size_t)NG * nn), sizeof(double));
    char *scr = nullptr;
    if ((st = arena_get(device, stream, need, &scr))) return st;
    Carve cv{scr};
    PixelRec *d_pix = cv.take<PixelRec>(n_pix);
    double2 *d_H = cv.take<double2>((size_t)CH * plane);
    double *d_img = cv.take<double>(fused ? 1 : (size_t)CH * nn);
    double2 *d_D = cv.take<double2>(CH);
    double *d_s1 = cv.take<double>((size_t)nn);
    double *d_s2 = cv.take<double>((size_t)nn);
    double *d_part = cv.take<double>(nb);
    double *d_loss = cv.take<double>(1);
    double *d_s1p = cv.take<double>(std::max<size_t>(1, (size_t)NG * nn));
    double *d_s2p = cv.take<double>(std::max<size_t>(1, (size_t)NG * nn));
    const double2 *d_tw = nullptr;
    const double *d_atan = nullptr;
    if (fused && ((st = twiddle_table_device(device, N, &d_tw)) || (st = atan_table_device(device, &d_atan))))
        return st;
    const ApertureDev apd = make_aperture_dev(optics);
    const OpticsDev opd = make_optics_dev(optics);
    HIP_TRY(launch_pixel_terms(L.d_pixbase, d_pix, n_pix, apd, opd, nullptr, 0, nullptr, stream));
    HIP_TRY(launch_fill_zero(d_s1, (size_t)nn, stream));
    HIP_TRY(launch_fill_zero(d_s2, (size_t)nn, stream));
    CorrParams cp;
    std::memset(&cp, 0, sizeof cp);
    cp.G = (const float2 *)G_c64_dev;
    cp.N = N;
    cp.nh = nh;
    cp.ldq = optics->wavelength_A / (N * scan->step_A);
    cp.ap = apd;
    cp.op = opd;
    cp.H = d_H;
    cp.D = d_D;
    if ((st = trig_table_device(device, &cp.trig))) return st;
    for (int c0 = 0; c0 < n_pix; c0 += CH) {
        const int cn = std::min(CH, n_pix - c0);
        cp.pix = d_pix + c0;
        cp.goff = L.d_goff + c0;
        cp.n_valid = cn;
        if (fused) {
            HIP_TRY(launch_loss_fused(cp, d_tw, d_atan, cn, L.d_pixbase + c0, std::min(NG, cn), d_s1p, d_s2p, d_s1, d_s2,
                                      stream));
            continue;
        }
        HIP_TRY(launch_corrected_half(cp, CH, stream));
        if ((st = fft_z2d(device, N, CH, d_H, d_img, stream))) return st;
        HIP_TRY(launch_phase_moments(d_img, d_D, L.d_pixbase + c0, cn, nn, d_s1, d_s2, stream));
    }
    HIP_TRY(launch_loss(d_s1, d_s2, nn, W, mean_phase_out_dev, d_part, d_loss, stream));
    if (loss_out_host) {
        HIP_TRY(hipMemcpyAsync(loss_out_host, d_loss, sizeof(double), hipMemcpyDeviceToHost, stream));
        HIP_TRY(hipStreamSynchronize(stream));
    }
    return DSP_OK;
}

dsp_status dsp_quantize_herm16(const void *G_c64_dev, int n_bf, int n_scan, int row_scales, void *Q_i16_dev,
                               float *scale_dev, void *hip_stream) {
    if (!G_c64_dev || !Q_i16_dev || !scale_dev) return fail(DSP_EINVAL, "G, Q and scale must be non-NULL");
    if (n_bf <= 0) return fail(DSP_EINVAL, "n_bf must be > 0");
    if (n_scan < 4 || (n_scan & 1)) return fail(DSP_EINVAL, "n_scan must be even and >= 4");
    // the pack kernel reads two entries per 16-byte load and writes them in one 8-byte store
    if ((uintptr_t)G_c64_dev % 16 || (uintptr_t)Q_i16_dev % 8)
        return fail(DSP_EINVAL, "G must be 16-byte and Q 8-byte aligned");
    HIP_TRY(launch_herm16((const float2 *)G_c64_dev, n_bf, n_scan, n_scan / 2 + 1, row_scales != 0,
                          (short2 *)Q_i16_dev, scale_dev, (hipStream_t)hip_stream));
    return DSP_OK;
}

}  // extern "C"
