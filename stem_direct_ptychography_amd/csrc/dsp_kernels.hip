// HIP kernels of libdsp for CDNA4 (gfx950, wave64).
//
// Regularized direct (single-side-band) ptychography, per scan frequency q:
// transfer T(q, k, alias) evaluated in registers, weighted augmented Gram
// [T g]^H W [T g] reduced over bright-field pixels in FP64, eigenbasis or
// solve per q, and the SSB sum over pixels ("Where the 9 s of regularized
// preparation goes", section "Code path"; "Preparation in one kernel per
// alias count", section "What changed"; "Tilt-corrected SSB on CUDA",
// section "Changes").
//
// Lane mapping of the streaming kernels: a wave owns a tile of up to 64 scan
// frequencies (one per lane, cut along G's 128-byte lines by the host) and
// walks the bright-field pixels in lockstep.  Per-pixel data (lambda k,
// sqrt(w) a(k), chi(k), plane offset) is wave-uniform and staged in LDS;
// each lane reads its own G(q, k); the lens-overlap zero-skip branches
// almost never diverge because neighbouring frequencies see nearly the same
// lens; each lane keeps its own frequency's sums, so there is no cross-lane
// reduction.  While a chunk of pixels is staged, a wave-uniform test against
// the tile's centre and radius marks the alias slots that no lane can have
// in support; they are skipped with scalar branches.  The upsampled preview
// runs the same kernel with right sides only: a lane's slots are the fine
// frequencies that read its stored G value ("Historical WebGPU G(q,k) memory
// experiment", section "Object-redraw fast path").  The tiles x pixels of a
// launch are split into equal-cost contiguous ranges (stream-K, costed per
// iteration by the same test on the host), eight per resident wave slot;
// partial sums are added per tile in a fixed order afterwards
// (deterministic).  A chunk's staging issues all of its loads before the
// first is used: vector loads complete in issue order, and a wait per load
// would expose each one's latency.
//
// The loss path takes each pixel's corrected half plane through an inverse
// real 2D transform in two fused passes, self-sorting radix-8 transforms in
// LDS: the column pass computes the corrected values itself, the row pass
// goes straight on to the phases and their moments.
#include "dsp_internal.hpp"
#include "dsp_kernels.hpp"

#include <cstring>
#include <algorithm>
#include <mutex>
#include <type_traits>

namespace dsp {

// ---------------------------------------------------------------------------
// shared device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool inside_support(const ApertureDev &ap, double d2) {
    return ap.soft ? (d2 < ap.rout2) : (d2 <= ap.rout2);
}

// a(k') for a point already known to be inside the support.
__device__ __forceinline__ double lobe_aperture(const ApertureDev &ap, double d2) {
    if (!ap.soft || d2 <= ap.rin2) return 1.0;
    return fma(ap.kc - sqrt(d2), ap.inv_dk, 0.5);
}

__device__ __forceinline__ double aperture_at(const ApertureDev &ap, double d2) {
    if (!inside_support(ap, d2)) return 0.0;
    return lobe_aperture(ap, d2);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

// sinc(h) = sin(h) / h of a lobe's depth term: the sine of sincos_tab and the
// hardware reciprocal refined by two Newton steps (relative error about
// 1e-16, in place of a correctly rounded division); the series below |h| =
// 1e-4 (error below 1e-28).
__device__ __forceinline__ double sinc_tab(double h, const double2 *__restrict__ T) {
    double sn, cs;
    sincos_tab(h, T, sn, cs);
    double r = __builtin_amdgcn_rcp(h);
    r = fma(r, fma(-h, r, 1.0), r);
    r = fma(r, fma(-h, r, 1.0), r);
    const double h2 = h * h;
    const double series = fma(h2, fma(h2, 1.0 / 120.0, -1.0 / 6.0), 1.0);
    return fabs(h) < 1e-4 ? series : sn * r;
}

// sqrt(d2) for the aperture's soft edge (Gram and SSB kernels): the FP32
// reciprocal square root (measured relative error 1e-7) refined by one
// Newton step in FP64, relative error about 1e-14.
__device__ __forceinline__ double sqrt_fast(double d2) {
    const double r = (double)__builtin_amdgcn_rsqf((float)d2);
    const double s0 = d2 * r;
    return fma(0.5 * r, fma(-s0, s0, d2), s0);
}

// The leading coefficients of chi's Horner rows (chi_poly_top) held in VGPRs:
// from scalar registers each row's first FMA would have two scalar operands
// and take a register copy per evaluation (the empty asm hides that the
// values are uniform).  Row 6's single coefficient stays scalar.
__device__ __forceinline__ void chi_tops(const double *c, double (&top)[CHI_DEG + 1]) {
#pragma unroll
    for (int j = 0; j <= CHI_DEG; ++j) {
        double v = c[chi_off(j) + CHI_DEG - j];
        if (j < CHI_DEG) asm volatile("" : "+v"(v));
        top[j] = v;
    }
}

// ---------------------------------------------------------------------------
// pixel terms: a(k) and chi(k) once per pixel and optics set
// ---------------------------------------------------------------------------

// in[p] -> out[p]: lambda k, sqrt(w) a(k) and chi(theta(k)), theta(k) =
// lambda k + tau formed as a rounded product then a rounded add (never
// fused), exactly as the Gram and SSB kernels form it; with chi_tab
// non-null, chi alone into chi_tab[p * chi_stride] (an SSB pass's sets);
// with tay non-null also chi's Taylor coefficients about theta(k) into
// tay[p * TAY_N] (the Gram kernels' lobe phases).
__global__ void pixel_terms_kernel(const PixelBase *in, PixelRec *out, int n_pix, ApertureDev ap, OpticsDev op,
                                   double *chi_tab, int chi_stride, double *tay) {
#pragma clang fp contract(off)
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_pix) return;
    const double ky = in[p].ky, kx = in[p].kx;
    const double lky = op.lam * ky, lkx = op.lam * kx;
    const double c = chi_poly(op.chi_c, lkx + op.tau_x, lky + op.tau_y);
    if (chi_tab) {
        chi_tab[(size_t)p * chi_stride] = c;
        return;
    }
    if (tay) {
        double t[TAY_N];
        chi_taylor(op.chi_c, lkx + op.tau_x, lky + op.tau_y, t);
#pragma unroll
        for (int m = 0; m < TAY_N; ++m) tay[(size_t)p * TAY_N + m] = t[m];
    }
    if (!out) return;   // Taylor coefficients only
    PixelRec r;
    r.lky = lky;
    r.lkx = lkx;
    r.amp0 = in[p].sw * aperture_at(ap, fma(ky, ky, kx * kx));
    r.sw = in[p].sw;
    r.chi0 = c;
    r.pad = 0.0;
    out[p] = r;
}

// ---------------------------------------------------------------------------
// transfer + weighted augmented Gram
// ---------------------------------------------------------------------------
// METHOD 0 (phase): columns T_phi(slot 0..NJ-1), then g.
// METHOD 1 (complex): columns L(slot 0..NJ-1), R(slot 0..NJ-1), then g; the
// write-out turns them into [T_A, T_phi] (T_A = L + R, T_phi = i (L - R)),
// which keeps the per-pixel update to the lobes actually present.
template <int NJ, int METHOD>
struct GramShape {
    static constexpr int NC = METHOD == 0 ? NJ : 2 * NJ;
    static constexpr int D = NC + 1;
    static constexpr int NOFF = D * (D - 1) / 2;
    static constexpr int NACC = D + 2 * NOFF;
    // strict upper index of (c, d), c < d
    static constexpr int off(int c, int d) { return c * (2 * D - c - 1) / 2 + (d - c - 1); }
    static constexpr int re(int c, int d) { return D + 2 * off(c, d); }
    static constexpr int im(int c, int d) { return D + 2 * off(c, d) + 1; }
};

// METHOD 2 (the upsampled preview): columns T_phi(slot 0..NJ-1), right
// sides only, conj(T_phi) w g per slot: two doubles per slot.
template <int NJ>
struct GramShape<NJ, 2> {
    static constexpr int NC = NJ;
    static constexpr int D = NC + 1;
    static constexpr int NOFF = 0;
    static constexpr int NACC = 2 * NJ;
    static constexpr int re(int c, int) { return 2 * c; }
    static constexpr int im(int c, int) { return 2 * c + 1; }
};

// Complex method: the sums of column pairs within one side (L x L and R x R,
// both columns below NJ or both in NJ .. 2 NJ - 1) live in LDS, one double2
// per pair and lane; they are updated least often, and keeping them out of
// the registers lets two waves share a SIMD.
template <int NJ, int METHOD>
struct GramLds {
    static constexpr int NH = NJ * (NJ - 1) / 2;              // pairs per side
    static constexpr int NP = METHOD == 1 ? 2 * NH : 0;
    static constexpr bool in_lds(int c, int d) {
        return METHOD == 1 && c < d && d < 2 * NJ && ((d < NJ) || (c >= NJ));
    }
    static constexpr int tri(int c, int d) { return c * (2 * NJ - c - 1) / 2 + (d - c - 1); }   // c < d < NJ
    static constexpr int idx(int c, int d) { return c < NJ ? tri(c, d) : NH + tri(c - NJ, d - NJ); }
};

template <int NJ, int METHOD>
__device__ __forceinline__ void acc_get(const double *acc, int c, int d, double &xr, double &xi) {
    using Sh = GramShape<NJ, METHOD>;
    // <col c, col d> for any order (compile-time indices after unrolling)
    if (c == d) {
        xr = acc[c];
        xi = 0.0;
    } else if (c < d) {
        xr = acc[Sh::re(c, d)];
        xi = acc[Sh::im(c, d)];
    } else {
        xr = acc[Sh::re(d, c)];
        xi = -acc[Sh::im(d, c)];
    }
}

// Write one frequency's augmented system (lane = frequency) from its sums.
template <int NJ, int METHOD>
__device__ __forceinline__ void write_system(const double *acc, unsigned mask, int qi, const GramParams &prm) {
    using Sh = GramShape<NJ, METHOD>;
    constexpr int NC = Sh::NC;
    const int Dout = prm.D;
    const int am = prm.a_max;
    double2 *out = prm.sys + (size_t)qi * (size_t)tri_size(Dout);
    for (int e = 0; e < tri_size(Dout); ++e) out[e] = make_double2(0.0, 0.0);
    bool act[NJ];
    int rank[NJ];
#pragma unroll
    for (int s = 0; s < NJ; ++s) {
        act[s] = (mask >> s) & 1u;
        rank[s] = __popc(mask & ((1u << s) - 1u));
    }
    const int gcol = Dout - 1;
    out[tri_idx(gcol, gcol, Dout)] = make_double2(acc[NC], 0.0);

    if (METHOD == 0) {
#pragma unroll
        for (int s = 0; s < NJ; ++s) {
            if (!act[s]) continue;
            const int i = rank[s];
            out[tri_idx(i, i, Dout)] = make_double2(acc[s], 0.0);
            out[tri_idx(i, gcol, Dout)] = make_double2(acc[Sh::re(s, NC)], acc[Sh::im(s, NC)]);
#pragma unroll
            for (int t = s + 1; t < NJ; ++t) {
                if (!act[t]) continue;
                out[tri_idx(i, rank[t], Dout)] = make_double2(acc[Sh::re(s, t)], acc[Sh::im(s, t)]);
            }
        }
    } else {
        // <L_s|L_t>, <L_s|R_t>, <R_s|L_t>, <R_s|R_t> -> [T_A, T_phi] blocks
#pragma unroll
        for (int s = 0; s < NJ; ++s) {
            if (!act[s]) continue;
            const int i = rank[s];
            double lgr, lgi, rgr, rgi;
            acc_get<NJ, METHOD>(acc, s, NC, lgr, lgi);
            acc_get<NJ, METHOD>(acc, NJ + s, NC, rgr, rgi);
            // <T_A s, g> = Lg + Rg;  <T_phi s, g> = -i (Lg - Rg)
            out[tri_idx(i, gcol, Dout)] = make_double2(lgr + rgr, lgi + rgi);
            out[tri_idx(am + i, gcol, Dout)] = make_double2(lgi - rgi, -(lgr - rgr));
#pragma unroll
            for (int t = 0; t < NJ; ++t) {
                if (!act[t]) continue;
                const int j = rank[t];
                double llr, lli, lrr, lri, rlr, rli, rrr, rri;
                acc_get<NJ, METHOD>(acc, s, t, llr, lli);
                acc_get<NJ, METHOD>(acc, s, NJ + t, lrr, lri);
                acc_get<NJ, METHOD>(acc, NJ + s, t, rlr, rli);
                acc_get<NJ, METHOD>(acc, NJ + s, NJ + t, rrr, rri);
                // <T_A s, T_phi t> = i (LL - LR + RL - RR): all (s, t)
                {
                    const double zr = llr - lrr + rlr - rrr, zi = lli - lri + rli - rri;
                    out[tri_idx(i, am + j, Dout)] = make_double2(-zi, zr);
                }
                if (t >= s) {
                    // <T_A s, T_A t> = LL + LR + RL + RR
                    const double ar = llr + lrr + rlr + rrr, ai = lli + lri + rli + rri;
                    // <T_phi s, T_phi t> = LL - LR - RL + RR
                    const double pr = llr - lrr - rlr + rrr, pi = lli - lri - rli + rri;
                    out[tri_idx(i, j, Dout)] = make_double2(ar, t == s ? 0.0 : ai);
                    out[tri_idx(am + i, am + j, Dout)] = make_double2(pr, t == s ? 0.0 : pi);
                }
            }
        }
    }
}

// Lobe-phase scheme of a Gram kernel (see gram_pixel).  The Taylor scheme
// saves about a third of a slot's lobe arithmetic but holds twenty more
// doubles per lane; it pays only where that costs no wave per SIMD (measured
// on the 512 x 512 full-frame prepare: 5-slot phase 2.73 -> 2.52 ms, 5-slot
// complex 5.16 -> 5.08 ms; the 4-slot phase kernel, pushed from three waves
// to two, went 8.43 -> 9.23 ms).
template <int NJ, int METHOD>
struct GramTaylor {
    static constexpr bool value = (METHOD == 1 && NJ >= 5);
};

// Pixels whose records (and, with the Taylor scheme, chi's coefficients
// about theta(k): 160 bytes each) are staged in LDS at a time.  16 for the
// 6-slot complex kernel keeps four of its blocks (30 KB of pair sums each)
// within a CU's 160 KB.
template <int NJ, int METHOD>
struct GramChunk {
    static constexpr int value = GramTaylor<NJ, METHOD>::value ? ((METHOD == 1 && NJ >= 6) ? 16 : 32) : 64;
};
constexpr int SSB_CHUNK = 64;

// G values fetched ahead per lane: one group of PF pixels (divides the chunk).
// Two for the phase kernels (no measurable loss, and it keeps the 4-slot
// kernel within three waves per SIMD without spills), four for complex.
template <int NJ, int METHOD>
struct GramPrefetch {
    static constexpr int value = METHOD == 1 ? 4 : 2;
};

// Waves per SIMD the compiler must fit (caps the registers per lane).
template <int NJ, int METHOD>
struct GramWaves {
    static constexpr int value = METHOD == 2   ? (NJ <= 5 ? 4 : 3)
                                 : METHOD == 0 ? (NJ <= 2 ? 4 : (NJ <= 4 ? 3 : (NJ <= 6 ? 2 : 1)))
                                               : (NJ <= 1 ? 4 : (NJ <= 2 ? 3 : (NJ <= 4 ? 2 : 1)));
};

// Pixel records and plane offsets are written by earlier kernels or copies,
// so they are read with ordinary (vector) loads: reading them through the
// constant address space (scalar loads) returned stale values when a freed
// buffer's address was reused by the next prepare.  Only the kernel
// arguments, which the host writes for each launch, go through scalar loads.
typedef const PixelRec ConstPixel;
typedef const long long ConstLong;

// Depth term of a lobe (the weak object spread evenly through the depth t
// below the plane chi refers to; "Where the 9 s of regularized preparation
// goes", What changed 2: "chi, sinc and phase factor"): with
// h = pi t (|theta_k|^2 - |theta'|^2) / (2 lambda) the lobe's phase argument
// chi(k) - chi(k') gains h and its amplitude is multiplied by sinc(h)
// (sinc_tab above).

// One lobe of the transfer at the pixel (amp0 = sqrt(w) a(k)) and the
// displaced point k' = k -/+ Q with d2 = |lambda k'|^2 (inside the support):
//   value = amp0 a(k') exp(i arg),
// arg = chi(k) - chi(k - Q) (L) or chi(k + Q) - chi(k) (R), plus the depth
// term h with DEPTH (the amplitude then gains sinc(h)).
// a(k') = 1 except in the soft edge ring; the square root runs only when some
// lane of the wave is in the ring (the empty asm keeps the compiler from
// computing it unconditionally).
template <bool DEPTH>
__device__ __forceinline__ void lobe(const GramParams &prm, const double2 *T, double arg, double h, double d2,
                                     double amp0, double &re, double &im) {
    double amp = amp0;
    if (DEPTH) amp *= sinc_tab(h, T);
    double sn, cs;
    sincos_tab(arg, T, sn, cs);
    const bool ring = d2 > prm.ap.lrin2;
    if (wave_any(ring)) {
        asm volatile("");
        if (ring) amp *= fma(prm.ap.lkc - sqrt_fast(d2), prm.ap.inv_ldk, 0.5);
    }
    re = amp * cs;
    im = amp * sn;
}

// One pixel's update of a lane's sums: the lobes of every slot, then the
// rank-one update of the augmented Gram.  pm (wave-uniform) holds two bits
// per slot, L and R, clear when no lane of the tile can have that lobe in
// support at this pixel; a slot with both clear is skipped whole (its
// columns are zero).
// Lobe phases, two schemes (GramTaylor picks one per kernel):
//  TAY: chi expanded about theta(k) (the pixel's Taylor coefficients, read
//       from LDS into registers once per pixel); one evaluation of the even
//       and odd parts in d = lambda Q serves both lobes of a slot;
//  else: the aberration polynomial at both displaced points, minus chi(k).
template <int NJ, int METHOD, bool DEPTH, bool TAY>
__device__ __forceinline__ void gram_pixel(const GramParams &prm, const double2 *T,
                                           double (&acc)[GramShape<NJ, METHOD>::NACC], double2 *lpair, int yh, int ix,
                                           const int (&jyN)[NJ], const int (&jxN)[NJ], const bool (&act)[NJ],
                                           unsigned pm, double lky, double lkx, double amp0, double sw,
                                           double chi0, const double *tay, float2 gv, const double *ctop) {
    using Sh = GramShape<NJ, METHOD>;
    constexpr int NC = Sh::NC;
    const double ldq = prm.ldq, lrlim2 = prm.ap.lrlim2;
    const double tau_y = prm.op.tau_y, tau_x = prm.op.tau_x;
    const double lk2 = fma(lky, lky, lkx * lkx);
    const double py = lky + tau_y, px = lkx + tau_x;   // theta(k)
    const double th0 = (DEPTH && !TAY) ? fma(px, px, py * py) : 0.0;
    double tc[TAY ? TAY_N : 1];
    if (TAY) {
#pragma unroll
        for (int m = 0; m < TAY_N; ++m) tc[m] = tay[m];
    }

    const double gr = (double)gv.x * sw, gi = (double)gv.y * sw;
    if (METHOD != 2) acc[NC] = fma(gr, gr, fma(gi, gi, acc[NC]));   // signal power w |g|^2

    double tr[NC], ti[NC];
    unsigned long long bal[NC];   // lanes whose column is non-zero
#pragma unroll
    for (int s = 0; s < NJ; ++s) {
        if (!((pm >> (2 * s)) & 3u)) {
            // no lane of the tile has either lobe of this slot in support
            bal[s] = 0ull;
            tr[s] = ti[s] = 0.0;
            if (METHOD == 1) {
                bal[NJ + s] = 0ull;
                tr[NJ + s] = ti[NJ + s] = 0.0;
            }
            continue;
        }
        const double Qy_s = (double)(yh + jyN[s]) * ldq, Qx_s = (double)(ix + jxN[s]) * ldq;
        // |lambda (k -/+ Q)|^2 = |lambda k|^2 + |lambda Q|^2 -/+ 2 (lambda k).(lambda Q)
        const double kq = fma(lky, Qy_s, lkx * Qx_s);
        const double q2 = fma(Qy_s, Qy_s, Qx_s * Qx_s);
        const double base = lk2 + q2;
        const double dm2 = fma(-2.0, kq, base);
        const double dp2 = fma(2.0, kq, base);
        const bool zl = act[s] && dm2 < lrlim2;
        const bool zr = act[s] && dp2 < lrlim2;
        double Lr = 0.0, Li = 0.0, Rr = 0.0, Ri = 0.0;
        if (TAY) {
            if (zl || zr) {
                // chi(theta -/+ d) - chi(theta) = E -/+ O with d = lambda Q
                const double X = Qx_s * Qx_s, Y = Qy_s * Qy_s;
                const double E = chi_even(tc, prm.op.chi_c, X, Y, Qx_s * Qy_s);
                const double O = chi_odd(tc + 8, Qx_s, Qy_s, X, Y);
                if (DEPTH) {
                    // |theta|^2 - |theta - d|^2 = 2 theta.d - |d|^2 (L),
                    // |theta + d|^2 - |theta|^2 = 2 theta.d + |d|^2 (R)
                    const double td2 = 2.0 * fma(py, Qy_s, px * Qx_s);
                    const double hl = prm.op.pt2 * (td2 - q2), hr = prm.op.pt2 * (td2 + q2);
                    if (zl) lobe<DEPTH>(prm, T, (O - E) + hl, hl, dm2, amp0, Lr, Li);
                    if (zr) lobe<DEPTH>(prm, T, (O + E) + hr, hr, dp2, amp0, Rr, Ri);
                } else {
                    if (zl) lobe<DEPTH>(prm, T, O - E, 0.0, dm2, amp0, Lr, Li);
                    if (zr) lobe<DEPTH>(prm, T, O + E, 0.0, dp2, amp0, Rr, Ri);
                }
            }
        } else {
            // L: chi(k) - chi(k - Q) (+ h); R: the negation of chi(k) - chi(k + Q) (+ h)
            if (zl) {
                const double ty = py - Qy_s, tx = px - Qx_s;
                double arg = chi0 - chi_poly_top(prm.op.chi_c, ctop, tx, ty), h = 0.0;
                if (DEPTH) {
                    h = prm.op.pt2 * (th0 - fma(tx, tx, ty * ty));
                    arg += h;
                }
                lobe<DEPTH>(prm, T, arg, h, dm2, amp0, Lr, Li);
            }
            if (zr) {
                const double ty = py + Qy_s, tx = px + Qx_s;
                double arg = chi0 - chi_poly_top(prm.op.chi_c, ctop, tx, ty), h = 0.0;
                if (DEPTH) {
                    h = prm.op.pt2 * (th0 - fma(tx, tx, ty * ty));
                    arg += h;
                }
                lobe<DEPTH>(prm, T, -arg, h, dp2, amp0, Rr, Ri);
            }
        }
        if (METHOD == 2) {
            // right side only, added as soon as the slot's column is known
            // (no column is kept for pairs): <col s, g> = conj(T_phi) g
            const double t_r = Ri - Li, t_i = Lr - Rr;
            acc[Sh::re(s, NC)] = fma(t_r, gr, fma(t_i, gi, acc[Sh::re(s, NC)]));
            acc[Sh::im(s, NC)] = fma(t_r, gi, fma(-t_i, gr, acc[Sh::im(s, NC)]));
        } else if (METHOD == 0) {
            tr[s] = Ri - Li;   // T_phi = i (L - R)
            ti[s] = Lr - Rr;
            bal[s] = __ballot(zl || zr);
        } else {
            tr[s] = Lr;
            ti[s] = Li;
            bal[s] = __ballot(zl);
            tr[NJ + s] = Rr;
            ti[NJ + s] = Ri;
            bal[NJ + s] = __ballot(zr);
        }
    }

    // Column c is updated when the slot test admits its lobe (phase: either
    // lobe) at this pixel: the bits are known at the pixel's start, so the
    // branch does not wait for the lobes, and columns that no lane has add
    // exact zeros.  Pairs held in registers then run without a test (a
    // branch costs more than their FMAs); pairs held in LDS, whose atomics
    // are dearer, run when some lane has both columns.
    if (METHOD == 2) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const unsigned bits = METHOD == 0 ? (pm >> (2 * c)) & 3u : (pm >> (c < NJ ? 2 * c : 2 * (c - NJ) + 1)) & 1u;
        if (!bits) continue;
        acc[c] = fma(tr[c], tr[c], fma(ti[c], ti[c], acc[c]));
        // right side <col c, g> = conj(t_c) g
        acc[Sh::re(c, NC)] = fma(tr[c], gr, fma(ti[c], gi, acc[Sh::re(c, NC)]));
        acc[Sh::im(c, NC)] = fma(tr[c], gi, fma(-ti[c], gr, acc[Sh::im(c, NC)]));
#pragma unroll
        for (int d = c + 1; d < NC; ++d) {
            if (GramLds<NJ, METHOD>::in_lds(c, d)) {
                if (!(bal[c] & bal[d])) continue;
                // LDS FP64 atomic adds without return: the wave does not wait
                // for a read of the running sum.  Each lane owns its address
                // and a wave's LDS operations run in issue order, so the sums
                // are deterministic.
                double *lp = (double *)(lpair + GramLds<NJ, METHOD>::idx(c, d) * 64);
                const double pr = fma(tr[c], tr[d], ti[c] * ti[d]);
                const double pim = fma(tr[c], ti[d], -(ti[c] * tr[d]));
                __hip_atomic_fetch_add(lp, pr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(lp + 1, pim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                acc[Sh::re(c, d)] = fma(tr[c], tr[d], fma(ti[c], ti[d], acc[Sh::re(c, d)]));
                acc[Sh::im(c, d)] = fma(tr[c], ti[d], fma(-ti[c], tr[d], acc[Sh::im(c, d)]));
            }
        }
    }
}

// Transfer + weighted augmented Gram over one wave's stream-K range.
// METHOD 0 (phase): columns T_phi(slot 0..NJ-1), then g.
// METHOD 1 (complex): columns L(slot 0..NJ-1), R(slot 0..NJ-1), then g; the
// write-out turns them into [T_A, T_phi] (T_A = L + R, T_phi = i (L - R)),
// which keeps the per-pixel update to the lobes actually present.
// Lane = frequency of the tile; pixel records are wave-uniform.
// While pixel p is used, G for p + 1 is in flight (its plane offset was read
// one pixel earlier) and the record of p + 1 and the offset of p + 2 load.
template <int NJ, int METHOD, bool DEPTH>
__global__ __launch_bounds__(64, (GramWaves<NJ, METHOD>::value)) void gram_kernel(GramParams prm) {
    using Sh = GramShape<NJ, METHOD>;
    constexpr int NC = Sh::NC;
    constexpr int NACC = Sh::NACC;

    constexpr int PF = GramPrefetch<NJ, METHOD>::value;
    constexpr bool TAY = GramTaylor<NJ, METHOD>::value;
    constexpr int GRAM_CHUNK = GramChunk<NJ, METHOD>::value;
    __shared__ double2 T[TRIG_N];
    __shared__ PixelRec srec[GRAM_CHUNK];
    __shared__ long long sgoff[GRAM_CHUNK + PF];
    __shared__ unsigned smask[GRAM_CHUNK];   // per pixel of the chunk: the slot test's L/R bits
    __shared__ double2 scent[NJ];             // lambda (c + j_s N dq) per slot, c the tile centre
    __shared__ double sthr;                   // the slot test's squared bound
    __shared__ double stay[TAY ? GRAM_CHUNK * TAY_N : 1];   // [pixel][TAY_N] chi about theta(k)
    constexpr int NP = GramLds<NJ, METHOD>::NP;
    __shared__ double2 lpair_all[(NP > 0 ? NP : 1) * 64];
    const int lane = threadIdx.x;
    for (int i = lane; i < TRIG_N; i += 64) T[i] = prm.trig[i];

    const int wv = blockIdx.x;
    const long long n_pix = prm.n_pix;
    long long it = prm.wbegin[wv];
    const long long end = prm.wbegin[wv + 1];
    int seg = prm.seg_off[wv];
    ConstPixel *pix = (ConstPixel *)prm.pix;
    ConstLong *goffs = (ConstLong *)prm.goff;
    const float2 *__restrict__ G = prm.G;
    // the leading chi coefficients of rows 0..5 in VGPRs: from scalar
    // registers each such row's first Horner FMA would have two scalar
    // operands and need a copy (the empty asm hides that the values are
    // uniform); row 6's single coefficient enters an FMA beside two VGPRs
    // (not with the Taylor scheme, which does not evaluate the polynomial,
    // nor in the three depth kernels where the 12 VGPRs would spill)
    constexpr bool TOPV = !TAY && !(DEPTH && ((METHOD == 1 && NJ == 4) || (METHOD == 2 && (NJ == 5 || NJ == 9))));
    double ctop[CHI_DEG + 1];
#pragma unroll
    for (int j = 0; j <= CHI_DEG; ++j) {
        double v = prm.op.chi_c[chi_off(j) + CHI_DEG - j];
        if (TOPV && j < CHI_DEG) asm volatile("" : "+v"(v));
        ctop[j] = v;
    }
    while (it < end) {
        const int t = (int)(it / n_pix);
        const int p0 = (int)(it - (long long)t * n_pix);
        const int p1 = (int)((end - it) < (n_pix - p0) ? p0 + (end - it) : n_pix);
        const GramTile *tile = prm.tiles + t;
        const int yh = tile->lyh[lane];
        const int ix = tile->lix[lane];
        const bool valid = tile->qidx[lane] >= 0;
        const unsigned mask = valid ? (unsigned)tile->mask[lane] : 0u;
        const int iy = yh < 0 ? yh + prm.N : yh;
        const long long lane_off = valid ? (long long)iy * prm.nh + ix : 0;

        // slot offsets (j_y N, j_x N); lambda Q is rebuilt from them per
        // pixel, which keeps eight doubles per slot out of the registers
        int jyN[NJ], jxN[NJ];
        bool act[NJ];
#pragma unroll
        for (int s = 0; s < NJ; ++s) {
            jyN[s] = (int)tile->jy[s] * prm.N;
            jxN[s] = (int)tile->jx[s] * prm.N;
            act[s] = (mask >> s) & 1u;
        }
        unsigned live = 0;   // slots some lane of the tile has
#pragma unroll
        for (int s = 0; s < NJ; ++s)
            if (__ballot(act[s])) live |= 1u << s;
        // Slot test: lane frequencies lie within rad of the tile centre c,
        // so a lobe of slot s can be in support at pixel k only if
        // |lambda k -/+ lambda (c + j_s N dq)| < lambda r + rad lambda dq;
        // sthr is that bound squared, widened by a part in 1e9 against
        // rounding.  The values go through LDS so that the chunk loop reads
        // them afresh instead of holding them in registers.
        if (lane < NJ) {
            scent[lane] = make_double2(((double)tile->cy + (double)((int)tile->jy[lane] * prm.N)) * prm.ldq,
                                       ((double)tile->cx + (double)((int)tile->jx[lane] * prm.N)) * prm.ldq);
        }
        if (lane == 0) {
            const double rr = sqrt(prm.ap.lrlim2) + (double)tile->rad * prm.ldq;
            sthr = rr * rr * (1.0 + 1e-9);
        }
        double acc[NACC];
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = 0.0;
        double2 *lpair = lpair_all + lane;   // this lane's LDS sums, stride 64
#pragma unroll
        for (int i = 0; i < NP; ++i) lpair[i * 64] = make_double2(0.0, 0.0);

        // Pixel records and plane offsets go through LDS a chunk of GRAM_CHUNK
        // pixels at a time, so the only global loads in the pixel loop are
        // the G values (vector loads complete in issue order: a record load
        // in the loop would wait for every older G load).  G is fetched a
        // group of PF pixels ahead: while group r0 is used from ga, the loads
        // of group r0 + PF go out into gb, and gb moves to ga at the group's
        // end, one group's work after issue.  A chunk's tail up to a multiple
        // of PF runs on zero records (amplitude, sqrt(w) and g all zero:
        // nothing is added); plane offsets past the segment are clamped to
        // its last pixel.
        float2 ga[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) ga[i] = G[goffs[p0 + i < p1 ? p0 + i : p1 - 1] + lane_off];
        for (int c0 = p0; c0 < p1; c0 += GRAM_CHUNK) {
            const int cn = (p1 - c0) < GRAM_CHUNK ? (p1 - c0) : GRAM_CHUNK;
            // the chunk's loads all go out before the first is used (a wait
            // per load would expose each one's latency): lane = pixel of the
            // chunk (zero records past the end), then the Taylor coefficients
            // and plane offsets, coalesced
            PixelRec rec;
            rec.lky = rec.lkx = rec.amp0 = rec.sw = rec.chi0 = rec.pad = 0.0;
            if (lane < cn) rec = pix[c0 + lane];
            constexpr int NTV = TAY ? (GRAM_CHUNK * TAY_N + 63) / 64 : 1;
            double tv[NTV];
            if (TAY) {
#pragma unroll
                for (int u = 0; u < NTV; ++u) {
                    const int i = lane + 64 * u;
                    tv[u] = i < cn * TAY_N ? prm.tay[(size_t)c0 * TAY_N + i] : 0.0;
                }
            }
            constexpr int NGO = (GRAM_CHUNK + PF + 63) / 64;
            long long gov[NGO];
#pragma unroll
            for (int u = 0; u < NGO; ++u) {
                const int i = lane + 64 * u;
                gov[u] = i < GRAM_CHUNK + PF ? goffs[c0 + i < p1 ? c0 + i : p1 - 1] : 0;
            }
            __syncthreads();   // the previous chunk's records are no longer read
            if (lane < GRAM_CHUNK) {
                srec[lane] = rec;
                const double thr = sthr;
                unsigned m = 0;
#pragma unroll
                for (int s = 0; s < NJ; ++s) {
                    if (!((live >> s) & 1u)) continue;
                    const double2 c = scent[s];
                    const double ly = rec.lky - c.x, lx = rec.lkx - c.y;
                    const double ry = rec.lky + c.x, rx = rec.lkx + c.y;
                    if (fma(ly, ly, lx * lx) < thr) m |= 1u << (2 * s);
                    if (fma(ry, ry, rx * rx) < thr) m |= 2u << (2 * s);
                }
                smask[lane] = m;
            }
            if (TAY) {
#pragma unroll
                for (int u = 0; u < NTV; ++u) {
                    const int i = lane + 64 * u;
                    if (i < GRAM_CHUNK * TAY_N) stay[i] = tv[u];
                }
            }
#pragma unroll
            for (int u = 0; u < NGO; ++u) {
                const int i = lane + 64 * u;
                if (i < GRAM_CHUNK + PF) sgoff[i] = gov[u];
            }
            __syncthreads();
            for (int r0 = 0; r0 < cn; r0 += PF) {
                float2 gb[PF];
#pragma unroll
                for (int k = 0; k < PF; ++k) gb[k] = G[sgoff[r0 + PF + k] + lane_off];
#pragma unroll
                for (int k = 0; k < PF; ++k) {
                    const int r = r0 + k;
                    const float2 gv = r < cn ? ga[k] : make_float2(0.0f, 0.0f);
                    const unsigned pm = prm.slot_test ? __builtin_amdgcn_readfirstlane(smask[r]) : ~0u;
                    gram_pixel<NJ, METHOD, DEPTH, TAY>(prm, T, acc, lpair, yh, ix, jyN, jxN, act, pm, srec[r].lky,
                                                       srec[r].lkx, srec[r].amp0, srec[r].sw, srec[r].chi0,
                                                       stay + (TAY ? r * TAY_N : 0), gv, ctop);
                }
#pragma unroll
                for (int k = 0; k < PF; ++k) ga[k] = gb[k];
            }
        }

        double *po = prm.partial + (size_t)seg * (NACC * 64);
#pragma unroll
        for (int i = 0; i < NACC; ++i) po[i * 64 + lane] = acc[i];
#pragma unroll
        for (int c = 0; c < GramShape<NJ, METHOD>::NC; ++c) {
#pragma unroll
            for (int d = c + 1; d < GramShape<NJ, METHOD>::NC; ++d) {
                if (!GramLds<NJ, METHOD>::in_lds(c, d)) continue;
                const double2 v = lpair[GramLds<NJ, METHOD>::idx(c, d) * 64];
                po[GramShape<NJ, METHOD>::re(c, d) * 64 + lane] = v.x;
                po[GramShape<NJ, METHOD>::im(c, d) * 64 + lane] = v.y;
            }
        }
        ++seg;
        it += p1 - p0;
    }
}

// Fixup, step 1: thread (tile t, accumulator i, lane) adds tile t's segment
// sums in iteration order and stores the total in the tile's first segment.
// Grid (ceil(NACC / 4), n_tiles) of 256-thread workgroups, four accumulators
// per workgroup; the loads of four segments go out together, the adds stay
// in segment order.
__global__ __launch_bounds__(256) void gram_reduce_kernel(GramParams prm, int nacc) {
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = blockIdx.y;
    if (i >= nacc) return;
    const int s0 = prm.seg_first[t], s1 = prm.seg_first[t + 1];
    const double *P = prm.partial + (size_t)i * 64 + lane;
    const size_t stride = (size_t)nacc * 64;
    double acc = 0.0;
    int sg = s0;
    for (; sg + 4 <= s1; sg += 4) {
        const double a0 = P[(size_t)sg * stride], a1 = P[(size_t)(sg + 1) * stride];
        const double a2 = P[(size_t)(sg + 2) * stride], a3 = P[(size_t)(sg + 3) * stride];
        acc += a0;
        acc += a1;
        acc += a2;
        acc += a3;
    }
    for (; sg < s1; ++sg) acc += P[(size_t)sg * stride];
    prm.partial[((size_t)s0 * nacc + i) * 64 + lane] = acc;
}

// Fixup, step 2: write each tile's systems from its reduced sums.
template <int NJ, int METHOD>
__global__ __launch_bounds__(64) void gram_write_kernel(GramParams prm) {
    using Sh = GramShape<NJ, METHOD>;
    constexpr int NACC = Sh::NACC;
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    const GramTile *tile = prm.tiles + t;
    const int qi = tile->qidx[lane];
    if (qi < 0) return;
    double acc[NACC];
    const double *pi = prm.partial + (size_t)prm.seg_first[t] * (NACC * 64);
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = pi[i * 64 + lane];
    if constexpr (METHOD == 2) {
        // preview: slot s of stored entry (yh, ix) is the fine frequency
        // K = (yh + jy N, ix + jx N); its sum goes to S(K) when Kx >= 0 and,
        // conjugated, to S(-K) otherwise (-K then reads G through the mirror
        // G(-q) = conj G(q)).  The host admits only slots whose target lies
        // in the computed part of the fine half plane; the range test here
        // keeps every store inside the plane regardless.
        const int M = prm.fine_M, mh = prm.fine_mh;
        const unsigned mask = (unsigned)tile->mask[lane];
#pragma unroll
        for (int s = 0; s < NJ; ++s) {
            if (!((mask >> s) & 1u)) continue;
            int Ky = (int)tile->lyh[lane] + (int)tile->jy[s] * prm.N;
            int Kx = (int)tile->lix[lane] + (int)tile->jx[s] * prm.N;
            double re = acc[GramShape<NJ, 2>::re(s, 0)], im = acc[GramShape<NJ, 2>::im(s, 0)];
            if (Kx < 0) {
                Ky = -Ky;
                Kx = -Kx;
                im = -im;
            }
            const int row = Ky < 0 ? Ky + M : Ky;
            if (row < 0 || row >= M || Kx >= mh) continue;
            prm.sys[(size_t)row * mh + Kx] = make_double2(re, im);
        }
    } else {
        write_system<NJ, METHOD>(acc, (unsigned)tile->mask[lane], qi, prm);
    }
}

// Work a Gram launch does per frequency, counted exactly per lane (not the
// wave-wide union the Gram kernel evaluates): instrumentation, run after the
// prepare's own kernels.  out[tile][0..4] = support tests (pixel, alias, lobe),
// non-zero lobes, non-zero columns, non-zero column pairs c < d, and
// (pixel, frequency) terms.  A phase column is non-zero when either lobe is;
// complex columns are the L and R lobes themselves.
template <int METHOD>
__global__ __launch_bounds__(64) void work_count_kernel(GramParams prm, unsigned long long *out) {
    const int lane = threadIdx.x & 63;
    const GramTile *tile = prm.tiles + blockIdx.x;
    const int yh = tile->lyh[lane];
    const int ix = tile->lix[lane];
    const bool valid = tile->qidx[lane] >= 0;
    const unsigned mask = valid ? (unsigned)tile->mask[lane] : 0u;
    const int nj = tile->nj;
    unsigned long long tests = 0, lobes = 0, cols = 0, pairs = 0, terms = 0;
    for (int p = 0; p < prm.n_pix; ++p) {
        const double lky = prm.pix[p].lky, lkx = prm.pix[p].lkx, lk2 = fma(lky, lky, lkx * lkx);
        unsigned long long nc = 0;
        for (int s = 0; s < nj; ++s) {
            if (!((mask >> s) & 1u)) continue;
            const double Qy = (double)(yh + (int)tile->jy[s] * prm.N) * prm.ldq;
            const double Qx = (double)(ix + (int)tile->jx[s] * prm.N) * prm.ldq;
            const double kq = fma(lky, Qy, lkx * Qx);
            const double base = lk2 + fma(Qy, Qy, Qx * Qx);
            const bool zl = fma(-2.0, kq, base) < prm.ap.lrlim2;
            const bool zr = fma(2.0, kq, base) < prm.ap.lrlim2;
            tests += 2;
            lobes += (zl ? 1 : 0) + (zr ? 1 : 0);
            if (METHOD == 0) nc += (zl || zr) ? 1 : 0;
            else nc += (zl ? 1 : 0) + (zr ? 1 : 0);
        }
        cols += nc;
        pairs += nc * (nc - 1) / 2;   // 0 when nc = 0 (unsigned wrap times 0)
        terms += valid ? 1 : 0;
    }
    unsigned long long v[5] = {tests, lobes, cols, pairs, terms};
#pragma unroll
    for (int i = 0; i < 5; ++i) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v[i] += __shfl_xor(v[i], off);
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 5; ++i) out[(size_t)blockIdx.x * 5 + i] = v[i];
    }
}

// ---------------------------------------------------------------------------
// phase system from a complex one
// ---------------------------------------------------------------------------
// Thread = (frequency, packed entry of the phase triangle).  Slot m of the
// phase system is the complex system's T_phi slot a_max + m; g is slot a_max
// in the phase system and 2 a_max in the complex one.
__global__ void phase_from_complex_kernel(const double2 *csys, double2 *psys, int am, int n_q) {
    const int Dp = am + 1, Dc = 2 * am + 1;
    const int T = tri_size(Dp);
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)n_q * T) return;
    const int q = (int)(idx / T);
    int rem = (int)(idx - (long long)q * T);
    int i = 0;
    while (rem >= Dp - i) {
        rem -= Dp - i;
        ++i;
    }
    const int j = i + rem;
    const int ci = i < am ? am + i : 2 * am, cj = j < am ? am + j : 2 * am;
    psys[idx] = csys[(size_t)q * tri_size(Dc) + tri_idx(ci, cj, Dc)];
}

// ---------------------------------------------------------------------------
// phase eigenbasis: cyclic complex Jacobi, one lane per frequency
// ---------------------------------------------------------------------------

template <int A>
__global__ __launch_bounds__(64) void eig_kernel(EigParams prm) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= prm.n) return;
    const int q = prm.qlist[t];
    const int D = prm.D;
    const double2 *S = prm.sys + (size_t)q * (size_t)tri_size(D);
    double sc[A];
#pragma unroll
    for (int i = 0; i < A; ++i) sc[i] = 1.0 / sqrt(prm.prior[(size_t)q * prm.a_max + i]);
    // upper triangle of C = D^-1/2 M D^-1/2
    double hr[A][A], hi[A][A], vr[A][A], vi[A][A];
#pragma unroll
    for (int i = 0; i < A; ++i) {
#pragma unroll
        for (int j = 0; j < A; ++j) {
            vr[i][j] = (i == j) ? 1.0 : 0.0;
            vi[i][j] = 0.0;
            hr[i][j] = 0.0;
            hi[i][j] = 0.0;
        }
    }
#pragma unroll
    for (int i = 0; i < A; ++i) {
#pragma unroll
        for (int j = i; j < A; ++j) {
            const double2 e = S[tri_idx(i, j, D)];
            hr[i][j] = e.x * sc[i] * sc[j];
            hi[i][j] = (i == j) ? 0.0 : e.y * sc[i] * sc[j];
        }
    }
    for (int sweep = 0; sweep < 16; ++sweep) {
        double off = 0.0, dia = 0.0;
#pragma unroll
        for (int i = 0; i < A; ++i) {
            dia += hr[i][i] * hr[i][i];
#pragma unroll
            for (int j = i + 1; j < A; ++j) off += hr[i][j] * hr[i][j] + hi[i][j] * hi[i][j];
        }
        const bool done = off <= 1e-34 * dia;
        if (__all(done)) break;
#pragma unroll
        for (int p = 0; p < A; ++p) {
#pragma unroll
            for (int qq = p + 1; qq < A; ++qq) {
                const double br = hr[p][qq], bi = hi[p][qq];
                const double a = hr[p][p], d = hr[qq][qq];
                // |b| and e^{i phi} = b / |b| from components scaled to
                // order one, so |e| = 1 to rounding even where b * b would
                // underflow.  A rotation is applied only where |b| is above
                // 2^-60 (|a| + |d|): below that it changes the eigenvalues by
                // less than the rounding of the convergence test, and a phase
                // factor taken from a tiny |b| would only add error to V.
                const double bm = fmax(fabs(br), fabs(bi));
                const double sbr = bm > 0.0 ? br / bm : 0.0, sbi = bm > 0.0 ? bi / bm : 0.0;
                const double sn = sqrt(sbr * sbr + sbi * sbi);
                const double bn = bm * sn;
                const bool rot = bn > 0x1p-60 * (fabs(a) + fabs(d)) && bn > 0.0;
                const double er = rot ? sbr / sn : 1.0, ei = rot ? sbi / sn : 0.0;   // e^{i phi}
                const double zeta = rot ? (d - a) / (2.0 * bn) : 0.0;
                double tt = 1.0 / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
                tt = zeta < 0.0 ? -tt : tt;
                tt = rot ? tt : 0.0;
                const double c = 1.0 / sqrt(1.0 + tt * tt), s = tt * c;
                // J = [[c, s], [-s e^{-i phi}, c e^{-i phi}]] on columns (p, qq)
                if (!rot) continue;   // negligible: left in place (below the convergence test)
                hr[p][p] = a - tt * bn;
                hr[qq][qq] = d + tt * bn;
                hr[p][qq] = 0.0;
                hi[p][qq] = 0.0;
#pragma unroll
                for (int r = 0; r < A; ++r) {
                    if (r == p || r == qq) continue;
                    // H[r][p], H[r][qq] from upper storage
                    double xpr, xpi, xqr, xqi;
                    if (r < p) { xpr = hr[r][p]; xpi = hi[r][p]; } else { xpr = hr[p][r]; xpi = -hi[p][r]; }
                    if (r < qq) { xqr = hr[r][qq]; xqi = hi[r][qq]; } else { xqr = hr[qq][r]; xqi = -hi[qq][r]; }
                    // e^{-i phi} H[r][qq]
                    const double yr = er * xqr + ei * xqi, yi = er * xqi - ei * xqr;
                    const double npr = c * xpr - s * yr, npi = c * xpi - s * yi;
                    const double nqr = s * xpr + c * yr, nqi = s * xpi + c * yi;
                    if (r < p) { hr[r][p] = npr; hi[r][p] = npi; } else { hr[p][r] = npr; hi[p][r] = -npi; }
                    if (r < qq) { hr[r][qq] = nqr; hi[r][qq] = nqi; } else { hr[qq][r] = nqr; hi[qq][r] = -nqi; }
                }
#pragma unroll
                for (int r = 0; r < A; ++r) {
                    const double xpr = vr[r][p], xpi = vi[r][p], xqr = vr[r][qq], xqi = vi[r][qq];
                    const double yr = er * xqr + ei * xqi, yi = er * xqi - ei * xqr;
                    vr[r][p] = c * xpr - s * yr;
                    vi[r][p] = c * xpi - s * yi;
                    vr[r][qq] = s * xpr + c * yr;
                    vi[r][qq] = s * xpi + c * yi;
                }
            }
        }
    }
    // ascending order: odd-even transposition sort of (lambda, column)
    double lam[A];
#pragma unroll
    for (int i = 0; i < A; ++i) lam[i] = hr[i][i];
#pragma unroll
    for (int pass = 0; pass < A; ++pass) {
#pragma unroll
        for (int i = pass & 1; i + 1 < A; i += 2) {
            const bool sw = lam[i] > lam[i + 1];
            const double l0 = lam[i], l1 = lam[i + 1];
            lam[i] = sw ? l1 : l0;
            lam[i + 1] = sw ? l0 : l1;
#pragma unroll
            for (int r = 0; r < A; ++r) {
                const double a0 = vr[r][i], a1 = vr[r][i + 1], b0 = vi[r][i], b1 = vi[r][i + 1];
                vr[r][i] = sw ? a1 : a0;
                vr[r][i + 1] = sw ? a0 : a1;
                vi[r][i] = sw ? b1 : b0;
                vi[r][i + 1] = sw ? b0 : b1;
            }
        }
    }
    // U = D^-1/2 V, c = V^H D^-1/2 r
    const int am = prm.a_max;
    double rr[A], ri[A];
#pragma unroll
    for (int i = 0; i < A; ++i) {
        const double2 e = S[tri_idx(i, D - 1, D)];
        rr[i] = e.x * sc[i];
        ri[i] = e.y * sc[i];
    }
    double *lo = prm.lam + (size_t)q * am;
    double2 *Uo = prm.U + (size_t)q * am * am;
    double2 *co = prm.c + (size_t)q * am;
    for (int j = 0; j < am; ++j) {
        lo[j] = 0.0;
        co[j] = make_double2(0.0, 0.0);
    }
    for (int e = 0; e < am * am; ++e) Uo[e] = make_double2(0.0, 0.0);
#pragma unroll
    for (int j = 0; j < A; ++j) {
        lo[j] = lam[j];
        double cr = 0.0, ci = 0.0;
#pragma unroll
        for (int r = 0; r < A; ++r) {
            // conj(V_rj) * (r_r / sqrt p_r)
            cr = fma(vr[r][j], rr[r], fma(vi[r][j], ri[r], cr));
            ci = fma(vr[r][j], ri[r], fma(-vi[r][j], rr[r], ci));
            Uo[r * am + j] = make_double2(vr[r][j] * sc[r], vi[r][j] * sc[r]);
        }
        co[j] = make_double2(cr, ci);
    }
}

// ---------------------------------------------------------------------------
// solves
// ---------------------------------------------------------------------------

template <int A>
__global__ __launch_bounds__(64) void solve_phase_kernel(SolveParams prm) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= prm.n) return;
    const int q = prm.qlist[t];
    const int am = prm.a_max;
    double lam[A], cr[A], ci[A], ur[A][A], ui[A][A];
#pragma unroll
    for (int j = 0; j < A; ++j) {
        lam[j] = prm.lam[(size_t)q * am + j];
        const double2 c = prm.c[(size_t)q * am + j];
        cr[j] = c.x;
        ci[j] = c.y;
#pragma unroll
        for (int r = 0; r < A; ++r) {
            const double2 u = prm.U[((size_t)q * am + r) * am + j];
            ur[r][j] = u.x;
            ui[r][j] = u.y;
        }
    }
    const double P = prm.sys[(size_t)q * tri_size(prm.D) + tri_idx(prm.D - 1, prm.D - 1, prm.D)].x;
    for (int s = 0; s < prm.S; ++s) {
        const double mu = prm.strengths[s] * prm.scale;
        double yr[A], yi[A];
        double xr_dot = 0.0, quad = 0.0;
#pragma unroll
        for (int j = 0; j < A; ++j) {
            const double inv = 1.0 / (lam[j] + mu);
            yr[j] = cr[j] * inv;
            yi[j] = ci[j] * inv;
            xr_dot += yr[j] * cr[j] + yi[j] * ci[j];
            quad += lam[j] * (yr[j] * yr[j] + yi[j] * yi[j]);
        }
        double2 *xo = prm.x + ((size_t)s * prm.n_q + q) * am;
#pragma unroll
        for (int r = 0; r < A; ++r) {
            double xr = 0.0, xi = 0.0;
#pragma unroll
            for (int j = 0; j < A; ++j) {
                xr = fma(ur[r][j], yr[j], fma(-ui[r][j], yi[j], xr));
                xi = fma(ur[r][j], yi[j], fma(ui[r][j], yr[j], xi));
            }
            xo[r] = make_double2(xr, xi);
        }
        for (int r = A; r < am; ++r) xo[r] = make_double2(0.0, 0.0);
        if (prm.resid) prm.resid[(size_t)s * prm.n_q + q] = P - 2.0 * xr_dot + quad;
    }
}

// frequencies without aliases: nothing to solve, x = 0, misfit = P
__global__ __launch_bounds__(64) void solve_empty_kernel(SolveParams prm, int n_comp) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= prm.n) return;
    const int q = prm.qlist[t];
    const double P = prm.sys[(size_t)q * tri_size(prm.D) + tri_idx(prm.D - 1, prm.D - 1, prm.D)].x;
    for (int s = 0; s < prm.S; ++s) {
        for (int c = 0; c < n_comp; ++c) {
            double2 *xo = prm.x + ((size_t)(s * n_comp + c) * prm.n_q + q) * prm.a_max;
            for (int m = 0; m < prm.a_max; ++m) xo[m] = make_double2(0.0, 0.0);
        }
        if (prm.resid) prm.resid[(size_t)s * prm.n_q + q] = P;
    }
}

// complex method: Cholesky of M + scale diag(lambda_A p, lambda_phi p), d = 2A
// Cholesky factor of one complex system (lower triangle, row i, col j <= i):
// in registers, or, for the 12 x 12 systems of six aliases (78 complex
// entries, more than the registers hold without spilling), in LDS, one
// column of entries per thread of a SOLVE_LDS_THREADS-thread block.
constexpr int SOLVE_LDS_THREADS = 32;
template <int A>
struct SolveInLds {
    static constexpr bool value = 2 * A >= 12;
};

template <int d, bool LDS>
struct CholFactor;
template <int d>
struct CholFactor<d, false> {
    double r[d][d], i[d][d];
    __device__ __forceinline__ void set(int a, int b, double x, double y) {
        r[a][b] = x;
        i[a][b] = y;
    }
    __device__ __forceinline__ double re(int a, int b) const { return r[a][b]; }
    __device__ __forceinline__ double im(int a, int b) const { return i[a][b]; }
};
template <int d>
struct CholFactor<d, true> {
    double2 *col;   // this thread's entries: col[e * SOLVE_LDS_THREADS]
    __device__ __forceinline__ static int e(int a, int b) { return (a * (a + 1) / 2 + b) * SOLVE_LDS_THREADS; }
    __device__ __forceinline__ void set(int a, int b, double x, double y) { col[e(a, b)] = make_double2(x, y); }
    __device__ __forceinline__ double re(int a, int b) const { return col[e(a, b)].x; }
    __device__ __forceinline__ double im(int a, int b) const { return col[e(a, b)].y; }
};

template <int A>
__global__ __launch_bounds__(64) void solve_complex_kernel(SolveParams prm) {
    constexpr int d = 2 * A;
    constexpr bool LDSF = SolveInLds<A>::value;
    __shared__ double2 lsh[LDSF ? d * (d + 1) / 2 * SOLVE_LDS_THREADS : 1];
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= prm.n) return;
    const int q = prm.qlist[t];
    const int am = prm.a_max;
    const int D = prm.D;
    const double2 *S0 = prm.sys + (size_t)q * (size_t)tri_size(D);
    int slot[d];
#pragma unroll
    for (int i = 0; i < A; ++i) {
        slot[i] = i;
        slot[A + i] = am + i;
    }
    double pr[d];
#pragma unroll
    for (int i = 0; i < A; ++i) {
        pr[i] = prm.prior[(size_t)q * am + i];
        pr[A + i] = pr[i];
    }
    double rr[d], ri[d];
#pragma unroll
    for (int i = 0; i < d; ++i) {
        const double2 e = S0[tri_idx(slot[i], D - 1, D)];
        rr[i] = e.x;
        ri[i] = e.y;
    }
    const double P = S0[tri_idx(D - 1, D - 1, D)].x;
    for (int s = 0; s < prm.S; ++s) {
        const double la = prm.strengths[2 * s] * prm.scale, lp = prm.strengths[2 * s + 1] * prm.scale;
        // With the factor in LDS, the system is re-read for each strength: an
        // opaque zero offset keeps the compiler from hoisting its 78 entries
        // out of the strength loop into registers (which would spill).
        const double2 *S = S0;
        if constexpr (LDSF) {
            long long zo = 0;
            asm volatile("" : "+v"(zo));
            S = S0 + zo;
        }
        // lower triangle L (row i, col j <= i) of the Cholesky factor
        CholFactor<d, LDSF> L;
        if constexpr (LDSF) {
            // the regularized system H (lower triangle, H_ij = conj(M[slot j][slot
            // i])) copied into the factor's storage by a rolled loop, one entry
            // at a time, then factored in place
            L.col = lsh + threadIdx.x;
#pragma unroll 1
            for (int i = 0; i < d; ++i) {
                const int si = i < A ? i : am + i - A;
#pragma unroll 1
                for (int j = 0; j <= i; ++j) {
                    const int sj = j < A ? j : am + j - A;
                    const double2 e = S[tri_idx(sj, si, D)];
                    const double dg = i == j ? (j < A ? la : lp) * prm.prior[(size_t)q * am + (j < A ? j : j - A)] : 0.0;
                    L.col[(i * (i + 1) / 2 + j) * SOLVE_LDS_THREADS] = make_double2(e.x + dg, i == j ? 0.0 : -e.y);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < d; ++j) {
            // H_jj - sum_k |L_jk|^2
            double hjj = LDSF ? L.re(j, j) : S[tri_idx(slot[j], slot[j], D)].x + (j < A ? la : lp) * pr[j];
#pragma unroll
            for (int k = 0; k < j; ++k) hjj -= L.re(j, k) * L.re(j, k) + L.im(j, k) * L.im(j, k);
            const double ljj = sqrt(hjj);
            const double inv = 1.0 / ljj;
            L.set(j, j, ljj, 0.0);
#pragma unroll
            for (int i = j + 1; i < d; ++i) {
                // H_ij (i > j) = conj(M[slot j][slot i])
                double zr, zi;
                if constexpr (LDSF) {
                    zr = L.re(i, j);
                    zi = L.im(i, j);
                } else {
                    const double2 e = S[tri_idx(slot[j], slot[i], D)];
                    zr = e.x;
                    zi = -e.y;
                }
#pragma unroll
                for (int k = 0; k < j; ++k) {
                    // L_ik conj(L_jk)
                    zr -= L.re(i, k) * L.re(j, k) + L.im(i, k) * L.im(j, k);
                    zi -= L.im(i, k) * L.re(j, k) - L.re(i, k) * L.im(j, k);
                }
                L.set(i, j, zr * inv, zi * inv);
            }
        }
        // forward L z = r, backward L^H x = z, x overwriting z in place
        double xr[d], xi[d];
#pragma unroll
        for (int i = 0; i < d; ++i) {
            double ar = rr[i], ai = ri[i];
#pragma unroll
            for (int k = 0; k < i; ++k) {
                ar -= L.re(i, k) * xr[k] - L.im(i, k) * xi[k];
                ai -= L.re(i, k) * xi[k] + L.im(i, k) * xr[k];
            }
            xr[i] = ar / L.re(i, i);
            xi[i] = ai / L.re(i, i);
        }
#pragma unroll
        for (int i = d - 1; i >= 0; --i) {
            double ar = xr[i], ai = xi[i];
#pragma unroll
            for (int k = i + 1; k < d; ++k) {
                // conj(L_ki) x_k
                ar -= L.re(k, i) * xr[k] + L.im(k, i) * xi[k];
                ai -= L.re(k, i) * xi[k] - L.im(k, i) * xr[k];
            }
            xr[i] = ar / L.re(i, i);
            xi[i] = ai / L.re(i, i);
        }
        double2 *xo = prm.x + ((size_t)(2 * s) * prm.n_q + q) * am;
        double2 *xo2 = prm.x + ((size_t)(2 * s + 1) * prm.n_q + q) * am;
#pragma unroll
        for (int i = 0; i < A; ++i) {
            xo[i] = make_double2(xr[i], xi[i]);
            xo2[i] = make_double2(xr[A + i], xi[A + i]);
        }
        for (int i = A; i < am; ++i) {
            xo[i] = make_double2(0.0, 0.0);
            xo2[i] = make_double2(0.0, 0.0);
        }
        if (prm.resid) {
            // P - 2 Re(x^H r) + x^H M x
            double xr_dot = 0.0, quad = 0.0;
#pragma unroll
            for (int i = 0; i < d; ++i) {
                xr_dot += xr[i] * rr[i] + xi[i] * ri[i];
                double mr = 0.0, mi = 0.0;
#pragma unroll
                for (int j = 0; j < d; ++j) {
                    double er, ei;
                    if (i <= j) {
                        const double2 e = S[tri_idx(slot[i], slot[j], D)];
                        er = e.x;
                        ei = i == j ? 0.0 : e.y;
                    } else {
                        const double2 e = S[tri_idx(slot[j], slot[i], D)];
                        er = e.x;
                        ei = -e.y;
                    }
                    mr += er * xr[j] - ei * xi[j];
                    mi += er * xi[j] + ei * xr[j];
                }
                quad += xr[i] * mr + xi[i] * mi;
            }
            prm.resid[(size_t)s * prm.n_q + q] = P - 2.0 * xr_dot + quad;
        }
    }
}

// ---------------------------------------------------------------------------
// fill, scatter, export
// ---------------------------------------------------------------------------

__global__ void fill_zero_kernel(double *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0.0;
}

__global__ void scatter_kernel(ScatterParams prm) {
    // one thread per (strength x component, frequency)
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)prm.SC * prm.n_q;
    if (t >= total) return;
    const int sc = (int)(t / prm.n_q);
    const int q = (int)(t % prm.n_q);
    const int A = prm.count[q];
    const int nf = prm.nf, nfh = nf / 2 + 1;
    for (int m = 0; m < A; ++m) {
        const int ky = prm.K[((size_t)q * prm.a_max + m) * 2];
        const int kx = prm.K[((size_t)q * prm.a_max + m) * 2 + 1];
        const double2 v = prm.x[((size_t)sc * prm.n_q + q) * prm.a_max + m];
        size_t o;
        double2 val;
        if (kx > 0 || (kx == 0 && ky >= 0)) {
            o = (size_t)((ky % nf + nf) % nf) * nfh + kx;
            val = v;
        } else {
            o = (size_t)(((-ky) % nf + nf) % nf) * nfh + (-kx);
            val = make_double2(v.x, -v.y);
        }
        prm.spec[(size_t)sc * nf * nfh + o] = val;
    }
}

__global__ void export_kernel(const double2 *sys, int n_q, int D, double2 *dense) {
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)n_q * D * D;
    if (t >= total) return;
    const int q = (int)(t / ((size_t)D * D));
    const int ij = (int)(t % ((size_t)D * D));
    const int i = ij / D, j = ij % D;
    const double2 *S = sys + (size_t)q * tri_size(D);
    double2 v;
    if (i <= j) {
        v = S[tri_idx(i, j, D)];
    } else {
        const double2 e = S[tri_idx(j, i, D)];
        v = make_double2(e.x, -e.y);
    }
    dense[t] = v;
}

// ---------------------------------------------------------------------------
// SSB / agreement pass
// ---------------------------------------------------------------------------

// Waves per SIMD the SSB kernel must fit.  Eight sets fit three in 168
// registers with 4-pixel chunks (11 KB of LDS).
template <int MAXB, int H16>
struct SsbWaves {
    static constexpr int value = MAXB <= 2 ? 4 : (MAXB <= 4 ? 2 : 3);
};

// SSB sums over one wave's stream-K range of (band tile, pixel) iterations;
// lane = stored frequency q (one alias, Q = q).  Per set b:
//   Gamma_b = T_phi(q, k; b) = i (L_b - R_b),
//   S_b += w conj(Gamma_b) g,  N_b += w |Gamma_b|^2,  and P += w |g|^2.
// The support, a(k -/+ q), G and the weight are shared by the sets; chi and
// its phase factor are per set.  Partial layout: [3b] Re S_b, [3b+1] Im S_b,
// [3b+2] N_b, [3 MAXB] P.
// H16: G comes as herm16 snorm16 pairs, unpacked as max(q / 32767, -1) s in
// FP64 at use; H16 = 1: one scale per pixel (staged with the pixel record);
// H16 = 2: one scale per stored row, fetched with G for the lane's row.
template <int MAXB, bool DEPTH, int H16>
__global__ __launch_bounds__(64, (SsbWaves<MAXB, H16>::value)) void ssb_kernel(SsbParams prm) {
    constexpr int NACC = 3 * MAXB + 1;
    constexpr int PF = 2;   // G fetched one group of PF pixels ahead (as in gram_kernel)
    using GT = typename std::conditional<H16 != 0, short2, float2>::type;
    __shared__ double2 T[TRIG_N];
    // both lobes' phases come from each set's chi Taylor coefficients about
    // theta(k), staged per chunk (chunks of 16 or 8 pixels keep the LDS within
    // the kernel's waves per SIMD)
    constexpr int CHK = MAXB <= 2 ? 16 : (MAXB <= 4 ? 8 : 4);
    __shared__ PixelRec srec[CHK];
    __shared__ long long sgoff[CHK + PF];
    __shared__ long long sgrow[H16 == 2 ? CHK + PF : 1];   // pixel index x N (row scales)
    __shared__ double stay[MAXB * CHK * TAY_N];   // [set][pixel][TAY_N]
    // With eight sets the chunk's Taylor coefficients are computed in the
    // staging step, one lane per (set, pixel), from the sets' chi and tilt
    // copied to LDS here: reading them from the tables made every tile's wave
    // fetch 1280 bytes per pixel and wait for them at each chunk (12.3 ->
    // 11.1 ms on the 512 x 512 band).  With four, the shift's registers cost
    // a wave per SIMD (5.3 -> 5.7 ms), so fewer sets read the tables.
    constexpr bool TAYIN = MAXB >= 8;
    constexpr int CSTR = CHI_NCOEF + 2;
    __shared__ double schi[TAYIN ? MAXB * CSTR : 1];   // [set]: chi's coefficients, tau_y, tau_x
    const int lane = threadIdx.x;
    for (int i = lane; i < TRIG_N; i += 64) T[i] = prm.trig[i];
    if (TAYIN && lane == 0) {
#pragma unroll
        for (int b = 0; b < MAXB; ++b) {
#pragma unroll
            for (int i = 0; i < CHI_NCOEF; ++i) schi[b * CSTR + i] = prm.chi_c[b][i];
            schi[b * CSTR + CHI_NCOEF] = prm.tau_y[b];
            schi[b * CSTR + CHI_NCOEF + 1] = prm.tau_x[b];
        }
    }

    const int wv = blockIdx.x;
    const long long n_pix = prm.n_pix;
    long long it = prm.wbegin[wv];
    const long long end = prm.wbegin[wv + 1];
    // wave-uniform: the partial sums' base stays in scalar registers
    int seg = __builtin_amdgcn_readfirstlane(prm.seg_off[wv]);
    ConstPixel *pix = (ConstPixel *)prm.pix;
    ConstLong *goffs = (ConstLong *)prm.goff;
    const GT *__restrict__ G = H16 ? (const GT *)prm.GQ : (const GT *)prm.G;
    const float *__restrict__ gsc = prm.gscale;

    // the range's first tile and pixel; every later segment starts the next
    // tile at its first pixel (one division per wave, none held in registers)
    int t = (int)(it / n_pix);
    int p0 = (int)(it - (long long)t * n_pix);
    while (it < end) {
        const int p1 = (int)((end - it) < (n_pix - p0) ? p0 + (end - it) : n_pix);
        const SsbTile *tile = prm.tiles + t;
        const int yh = tile->lyh[lane];   // the lane's stored frequency q (signed row, column)
        const int ix = tile->lix[lane];
        const bool valid = (tile->valid >> lane) & 1ull;
        const int iyq = yh < 0 ? yh + prm.N : yh;   // its row in the stored half plane
        const long long lane_off = valid ? (long long)iyq * prm.nh + ix : 0;
        const double qy = (double)yh * prm.ldq, qx = (double)ix * prm.ldq;   // lambda q
        const double q2 = fma(qy, qy, qx * qx);
        const double qX = qx * qx, qY = qy * qy, qZ = qx * qy;   // powers of d = lambda q

        double acc[NACC];
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = 0.0;

        // records, plane offsets and the sets' Taylor coefficients staged in
        // LDS per chunk; G a group of PF pixels ahead; the chunk's tail runs on
        // zero records
        GT ga[PF];
        float sa[PF];   // row scales of the group (H16 == 2)
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const long long go = goffs[p0 + i < p1 ? p0 + i : p1 - 1];
            ga[i] = G[go + lane_off];
            if (H16 == 2) sa[i] = gsc[(go / prm.plane) * prm.N + iyq];
        }
        for (int c0 = p0; c0 < p1; c0 += CHK) {
            const int cn = (p1 - c0) < CHK ? (p1 - c0) : CHK;
            // the chunk's loads all go out before the first is used (a wait
            // per load would expose each one's latency): lane = pixel of the
            // chunk (zero records past the end; herm16: the pixel's scale
            // rides in the record's spare field), the sets' Taylor tables or,
            // with TAYIN, lane (set b, pixel c)'s lambda k, and the plane
            // offsets (CHK + PF <= 64: one per lane)
            PixelRec rec;
            rec.lky = rec.lkx = rec.amp0 = rec.sw = rec.chi0 = rec.pad = 0.0;
            if (lane < cn) rec = pix[c0 + lane];
            const long long go = goffs[c0 + lane < p1 ? c0 + lane : p1 - 1];
            float sc1 = 0.0f;
            if (H16 == 1 && lane < cn) sc1 = gsc[go / prm.plane];
            constexpr int NTV = TAYIN ? 1 : (CHK * TAY_N + 63) / 64;
            double tv[MAXB][NTV];
            double tky = 0.0, tkx = 0.0;
            const int tb_ = lane / CHK, tc_ = lane - tb_ * CHK;   // TAYIN: lane = (set, pixel)
            const bool tin = TAYIN && lane < MAXB * CHK && tb_ < prm.B && tc_ < cn;
            if (TAYIN) {
                if (tin) {
                    tky = pix[c0 + tc_].lky;
                    tkx = pix[c0 + tc_].lkx;
                }
            } else {
                // set b's table starts at b n_pix TAY_N
#pragma unroll
                for (int b = 0; b < MAXB; ++b) {
                    const double *tb = prm.tay + ((size_t)b * prm.n_pix + c0) * TAY_N;
#pragma unroll
                    for (int u = 0; u < NTV; ++u) {
                        const int i = lane + 64 * u;
                        tv[b][u] = (b < prm.B && i < cn * TAY_N) ? tb[i] : 0.0;
                    }
                }
            }
            __syncthreads();   // the previous chunk's LDS is no longer read
            if (H16 == 1) rec.pad = (double)sc1;
            if (lane < CHK) srec[lane] = rec;
            if (TAYIN) {
                // theta(k) = lambda k + tau formed as in the pixel-terms kernel
                // (a rounded add)
                if (lane < MAXB * CHK) {
                    double *ts = stay + (tb_ * CHK + tc_) * TAY_N;   // written in place
                    if (tin) {
                        const double *cb = schi + tb_ * CSTR;
                        chi_taylor(cb, tkx + cb[CHI_NCOEF + 1], tky + cb[CHI_NCOEF], ts);
                    } else {
#pragma unroll
                        for (int m = 0; m < TAY_N; ++m) ts[m] = 0.0;
                    }
                }
            } else {
#pragma unroll
                for (int b = 0; b < MAXB; ++b) {
#pragma unroll
                    for (int u = 0; u < NTV; ++u) {
                        const int i = lane + 64 * u;
                        if (i < CHK * TAY_N) stay[b * CHK * TAY_N + i] = tv[b][u];
                    }
                }
            }
            if (lane < CHK + PF) {
                sgoff[lane] = go;
                if (H16 == 2) sgrow[lane] = (go / prm.plane) * prm.N;
            }
            __syncthreads();
            for (int r0 = 0; r0 < cn; r0 += PF) {
                GT gb[PF];
                float sb[PF];
#pragma unroll
                for (int k = 0; k < PF; ++k) {
                    gb[k] = G[sgoff[r0 + PF + k] + lane_off];
                    if (H16 == 2) sb[k] = gsc[sgrow[r0 + PF + k] + iyq];
                }
#pragma unroll
                for (int k = 0; k < PF; ++k) {
                    const int r = r0 + k;
                    const double lky = srec[r].lky, lkx = srec[r].lkx, amp0 = srec[r].amp0, sw = srec[r].sw;
                    double gre, gim;   // G(q, k) in FP64
                    if (H16) {
                        const double sc = H16 == 1 ? srec[r].pad : (double)sa[k];
                        gre = fmax((double)ga[k].x * (1.0 / 32767.0), -1.0) * sc;
                        gim = fmax((double)ga[k].y * (1.0 / 32767.0), -1.0) * sc;
                    } else {
                        gre = (double)ga[k].x;
                        gim = (double)ga[k].y;
                    }
                    // (the chunk's tail, r >= cn, runs on zero records: sw = amp0 = 0
                    // zero its terms)
                    // Straight-line: nearly every pixel has both lobes in
                    // reach of some lane of the tile, so both are always evaluated
                    // for every set and a lane's lobe outside the support gets
                    // amplitude 0 by select (no per-lane branches, whose joins cost
                    // register copies, and no exec-mask bookkeeping).
                    const double lrlim2 = prm.ap.lrlim2, lrin2 = prm.ap.lrin2, lkc = prm.ap.lkc;
                    const double inv_ldk = prm.ap.inv_ldk;
                    const int B = prm.B;
                    const double lk2 = fma(lky, lky, lkx * lkx);
                    const double gr = gre * sw, gi = gim * sw;
                    acc[NACC - 1] = fma(gr, gr, fma(gi, gi, acc[NACC - 1]));
                    const double kq = fma(lky, qy, lkx * qx);
                    const double base = lk2 + q2;
                    const double dm2 = fma(-2.0, kq, base), dp2 = fma(2.0, kq, base);
                    const bool zl = valid && dm2 < lrlim2;
                    const bool zr = valid && dp2 < lrlim2;
                    double aml = zl ? amp0 : 0.0, amr = zr ? amp0 : 0.0;
                    const bool rl = zl && dm2 > lrin2, rr = zr && dp2 > lrin2;
                    if (wave_any(rl || rr)) {
                        const double fl = fma(lkc - sqrt_fast(dm2), inv_ldk, 0.5);
                        const double fr = fma(lkc - sqrt_fast(dp2), inv_ldk, 0.5);
                        aml = rl ? aml * fl : aml;
                        amr = rr ? amr * fr : amr;
                    }
#pragma unroll
                    for (int b = 0; b < MAXB; ++b) {
                        if (b >= B) continue;   // uniform; keeps the loop fully unrolled
                        int zb = 0;
                        // The set's coefficients are read from the kernel arguments
                        // per use (scalar loads, constant cache): an opaque zero
                        // offset keeps the compiler from hoisting all sets' values
                        // into scalar registers, which would spill.
                        if (MAXB > 1) asm volatile("" : "+s"(zb));
                        const double *cb = &prm.chi_c[b][zb];
                        // the even part's 8 coefficients, then the odd part's 12: the
                        // empty asm keeps the second group's LDS reads after the first
                        // evaluation, so fewer coefficients are live at once
                        const double *ts = stay + (b * CHK + r) * TAY_N;
                        double te[8], to[12];
#pragma unroll
                        for (int m = 0; m < 8; ++m) te[m] = ts[m];
                        const double E = chi_even(te, cb, qX, qY, qZ);
                        asm volatile("" ::: "memory");
#pragma unroll
                        for (int m = 0; m < 12; ++m) to[m] = ts[8 + m];
                        const double O = chi_odd(to, qx, qy, qX, qY);
                        double hl = 0.0, hr = 0.0, al = aml, ar = amr;
                        if (DEPTH) {
                            const double py = lky + prm.tau_y[b], px = lkx + prm.tau_x[b];
                            const double td2 = 2.0 * fma(py, qy, px * qx);
                            hl = prm.pt2[b] * (td2 - q2);
                            hr = prm.pt2[b] * (td2 + q2);
                            al *= sinc_tab(hl, T);
                            ar *= sinc_tab(hr, T);
                        }
                        double sl, cl, sr, cr;
                        // (without depth no + 0.0: IEEE's signed zero keeps the
                        // compiler from dropping it)
                        sincos_tab(DEPTH ? (O - E) + hl : O - E, T, sl, cl);
                        sincos_tab(DEPTH ? (O + E) + hr : O + E, T, sr, cr);
                        // Gamma = i (L - R); S += conj(Gamma) g'; N += |Gamma|^2
                        const double gmr = fma(ar, sr, -(al * sl)), gmi = fma(al, cl, -(ar * cr));
                        acc[3 * b] = fma(gmr, gr, fma(gmi, gi, acc[3 * b]));
                        acc[3 * b + 1] = fma(gmr, gi, fma(-gmi, gr, acc[3 * b + 1]));
                        acc[3 * b + 2] = fma(gmr, gmr, fma(gmi, gmi, acc[3 * b + 2]));
                    }
                }
#pragma unroll
                for (int k = 0; k < PF; ++k) {
                    ga[k] = gb[k];
                    if (H16 == 2) sa[k] = sb[k];
                }
            }
        }
        // the lane's offset is formed here (the empty asm keeps the compiler
        // from holding a 64-bit address across the pixel loop)
        double *po = prm.partial + (size_t)seg * (NACC * 64);
        int lo = lane;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int i = 0; i < NACC; ++i) po[i * 64 + lo] = acc[i];
        ++seg;
        it += p1 - p0;
        ++t;
        p0 = 0;
    }
}

// ---------------------------------------------------------------------------
// herm16 compact G ("Historical WebGPU G(q,k) memory experiment", compact
// preview): one scale per pixel, the largest |G| over its half plane, and
// each component packed as floor(0.5 + 32767 clamp(v / s, -1, 1)).
// ---------------------------------------------------------------------------

// Block = one pixel's plane: |G|^2 as a rounded sum of rounded squares in
// FP64, an exact max tree, the root rounded to float.
__device__ __forceinline__ double herm16_mag2(float re, float im) {
    const double r = re, i = im;
    return __dadd_rn(__dmul_rn(r, r), __dmul_rn(i, i));
}

// One scale per pixel plane (a block per plane): pairs of entries per 16-byte
// load (a plane holds N (N/2 + 1) entries, an even count, so pairs never
// straddle planes and stay aligned), four loads in flight per thread; the
// maximum is order-independent.
__global__ __launch_bounds__(256) void herm16_scale_kernel(const float2 *G, long long plane, float *scale) {
    __shared__ double red[256];
    const float4 *Gp = (const float4 *)(G + (size_t)blockIdx.x * plane);
    const long long npair = plane / 2;
    double m = 0.0;
    for (long long j = threadIdx.x; j < npair; j += 4 * 256) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = j + u * 256 < npair ? Gp[j + u * 256] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 4; ++u) m = fmax(m, fmax(herm16_mag2(v[u].x, v[u].y), herm16_mag2(v[u].z, v[u].w)));
    }
    red[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    if (threadIdx.x == 0) scale[blockIdx.x] = (float)sqrt(red[0]);
}

// One scale per stored row: wave w of the block takes row 4 b + w and its
// lanes the row's entries; the maximum is order-independent.
__global__ __launch_bounds__(256) void herm16_row_scale_kernel(const float2 *G, long long n_rows, int nh,
                                                                float *scale) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n_rows) return;
    const float2 *Gr = G + (size_t)row * nh;
    double m = 0.0;
    for (int e = lane; e < nh; e += 4 * 64) {
        float2 v[4];   // four loads in flight per lane
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = e + u * 64 < nh ? Gr[e + u * 64] : make_float2(0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 4; ++u) m = fmax(m, herm16_mag2(v[u].x, v[u].y));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    if (lane == 0) scale[row] = (float)sqrt(m);
}

// One entry's codes (the reading the oracle fixes: FP64 quotient, clamp,
// floor(0.5 + 32767 x); a zero scale packs zeros).
__device__ __forceinline__ unsigned herm16_code(float re, float im, double s) {
#pragma clang fp contract(off)
    if (!(s > 0.0)) return 0u;
    const double x = fmin(fmax((double)re / s, -1.0), 1.0), y = fmin(fmax((double)im / s, -1.0), 1.0);
    const short qx = (short)floor(0.5 + 32767.0 * x), qy = (short)floor(0.5 + 32767.0 * y);
    return (unsigned)(unsigned short)qx | ((unsigned)(unsigned short)qy << 16);
}

// Per-row scales and codes in one pass over G, for rows of at most 64
// HERM16_RPL entries: wave w of the block takes row 4 b + w, its lanes the
// row's entries, loaded once into registers; the row's largest |G|^2 by a
// wave reduction (the maximum is order-independent), then each lane's codes
// from its registers.  The same scale and codes as the two-pass form.
constexpr int HERM16_RPL = 9;   // entries per lane: rows of up to 576 entries (N <= 1024)
__global__ __launch_bounds__(256) void herm16_rows_fused_kernel(const float2 *G, long long n_rows, int nh,
                                                                float *scale, short2 *Q) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n_rows) return;   // whole waves
    const float2 *Gr = G + (size_t)row * nh;
    float2 v[HERM16_RPL];
    double m = 0.0;
#pragma unroll
    for (int u = 0; u < HERM16_RPL; ++u) {
        const int e = lane + 64 * u;
        v[u] = e < nh ? Gr[e] : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < HERM16_RPL; ++u) m = fmax(m, herm16_mag2(v[u].x, v[u].y));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    const float sc = (float)sqrt(m);
    if (lane == 0) scale[row] = sc;
    unsigned *Qr = (unsigned *)(Q + (size_t)row * nh);
#pragma unroll
    for (int u = 0; u < HERM16_RPL; ++u) {
        const int e = lane + 64 * u;
        if (e < nh) Qr[e] = herm16_code(v[u].x, v[u].y, (double)sc);
    }
}

// Block row y (grid-stride) takes pixel plane p; its threads take pairs of
// entries (one 16-byte load, one 8-byte store: a plane holds N (N/2 + 1)
// entries, an even count, so pairs never straddle planes and stay aligned).
// With row scales an entry e of the plane uses row e / nh's scale.
template <bool ROWS>
__global__ __launch_bounds__(256) void herm16_pack_kernel(const float2 *G, long long plane, int N, int nh, int n_bf,
                                                          const float *scale, short2 *Q) {
    const long long npair = plane / 2;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (int p = blockIdx.y; p < n_bf; p += gridDim.y) {
        const float4 *Gp = (const float4 *)(G + (size_t)p * plane);
        uint2 *Qp = (uint2 *)(Q + (size_t)p * plane);
        const double sp = ROWS ? 0.0 : (double)scale[p];
        const float *srow = scale + (size_t)p * N;
        // two pairs per thread and step, both loaded before either is coded
        for (long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x; j < npair; j += 2 * stride) {
            float4 v[2];
            double s0[2], s1[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const long long jj = j + u * stride;
                v[u] = jj < npair ? Gp[jj] : make_float4(0.f, 0.f, 0.f, 0.f);
                s0[u] = s1[u] = sp;
                if (ROWS && jj < npair) {
                    const unsigned e = (unsigned)(2 * jj);
                    s0[u] = (double)srow[e / (unsigned)nh];
                    s1[u] = (double)srow[(e + 1u) / (unsigned)nh];
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const long long jj = j + u * stride;
                if (jj < npair) Qp[jj] = make_uint2(herm16_code(v[u].x, v[u].y, s0[u]), herm16_code(v[u].z, v[u].w, s1[u]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// preview: DC term, spectrum and phase image
// ---------------------------------------------------------------------------
// dc = sum_k w_k G(0, k) over the active pixels: thread t adds pixels t,
// t + 256, ... in order, then a fixed tree (one block; deterministic).
__global__ __launch_bounds__(256) void preview_dc_kernel(const PixelBase *pix, const long long *goff, int n_pix,
                                                          const float2 *G, double2 *dc) {
    __shared__ double sr[256], si[256];
    double ar = 0.0, ai = 0.0;
    for (int p = threadIdx.x; p < n_pix; p += 256) {
        const float2 g = G[goff[p]];
        ar = fma(pix[p].w, (double)g.x, ar);
        ai = fma(pix[p].w, (double)g.y, ai);
    }
    sr[threadIdx.x] = ar;
    si[threadIdx.x] = ai;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) {
            sr[threadIdx.x] += sr[threadIdx.x + h];
            si[threadIdx.x] += si[threadIdx.x + h];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) dc[0] = make_double2(sr[0], si[0]);
}

// P(K) = i S(K) for K != 0, P(0) = dc (grid-stride over the half plane).
__global__ __launch_bounds__(256) void preview_spectrum_kernel(const double2 *S, const double2 *dc, long long n,
                                                                double2 *P) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
        const double2 v = S[e];
        P[e] = e == 0 ? dc[0] : make_double2(-v.y, v.x);
    }
}

// img[r] holds sum_{K != 0} S(K) e^{2 pi i K.r / M} (the unnormalized
// inverse real transform); the object is M^2 o(r) = dc + i img[r], so its
// phase is atan2(img[r] + Im dc, Re dc).
__global__ __launch_bounds__(256) void preview_phase_kernel(double *img, long long n, const double2 *dc) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    const double2 d = dc[0];
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride)
        img[e] = atan2(img[e] + d.y, d.x);
}

// ---------------------------------------------------------------------------
// loss path: per-pixel corrected planes, phase moments
// ---------------------------------------------------------------------------
// Block (x, j): 256 stored frequencies q of chunk pixel j.  Pixel k's object
// is C_k(0) + i (inverse real transform of H_k) up to the positive factor
// sqrt(w_k), which the phase does not see: H_k(q) = conj(Gamma'(q, k)) G(q, k)
// with Gamma' = sqrt(w) Gamma = i (L - R) built on amp0 = sqrt(w) a(k), and
// D_k = sqrt(w) G(0, k).  H is 0 at DC and on the Nyquist row and column.
// H_k(q) at stored entry (iy, ix) != DC, off the Nyquist row and column,
// for the pixel record rec and its stored value gv.
__device__ __forceinline__ double2 corrected_value(const CorrParams &prm, const double2 *T, const double *ctop,
                                                   const PixelRec &rec, float2 gv, int iy, int ix) {
    const int N = prm.N;
    const int yh = iy < N / 2 ? iy : iy - N;
    const double qy = (double)yh * prm.ldq, qx = (double)ix * prm.ldq;   // lambda q
    const double lky = rec.lky, lkx = rec.lkx;
    const double lk2 = fma(lky, lky, lkx * lkx);
    const double q2 = fma(qy, qy, qx * qx);
    const double kq = fma(lky, qy, lkx * qx);
    const double base = lk2 + q2;
    const double dm2 = fma(-2.0, kq, base), dp2 = fma(2.0, kq, base);
    const bool zl = dm2 < prm.ap.lrlim2, zr = dp2 < prm.ap.lrlim2;
    const double py = lky + prm.op.tau_y, px = lkx + prm.op.tau_x;   // theta(k), as chi0 was formed
    const bool depth = prm.op.pt2 != 0.0;
    const double th0 = fma(px, px, py * py);
    double Lr = 0.0, Li = 0.0, Rr = 0.0, Ri = 0.0;
    if (zl) {
        double a = rec.amp0;
        if (dm2 > prm.ap.lrin2) a *= fma(prm.ap.lkc - sqrt_fast(dm2), prm.ap.inv_ldk, 0.5);
        const double ty = py - qy, tx = px - qx;
        double arg = rec.chi0 - chi_poly_top(prm.op.chi_c, ctop, tx, ty);
        if (depth) {
            const double h = prm.op.pt2 * (th0 - fma(tx, tx, ty * ty));
            arg += h;
            a *= sinc_tab(h, T);
        }
        double sn, cs;
        sincos_tab(arg, T, sn, cs);
        Lr = a * cs;
        Li = a * sn;
    }
    if (zr) {
        double a = rec.amp0;
        if (dp2 > prm.ap.lrin2) a *= fma(prm.ap.lkc - sqrt_fast(dp2), prm.ap.inv_ldk, 0.5);
        const double ty = py + qy, tx = px + qx;
        double arg = rec.chi0 - chi_poly_top(prm.op.chi_c, ctop, tx, ty);
        if (depth) {
            const double h = prm.op.pt2 * (th0 - fma(tx, tx, ty * ty));
            arg += h;
            a *= sinc_tab(h, T);
        }
        double sn, cs;
        sincos_tab(-arg, T, sn, cs);
        Rr = a * cs;
        Ri = a * sn;
    }
    const double gmr = Ri - Li, gmi = Lr - Rr;   // Gamma' = i (L - R)
    const double gr = gv.x, gi = gv.y;
    return make_double2(fma(gmr, gr, gmi * gi), fma(gmr, gi, -(gmi * gr)));
}

__global__ __launch_bounds__(256) void corrected_half_kernel(CorrParams prm) {
    __shared__ double2 T[TRIG_N];
    if (threadIdx.x < TRIG_N) T[threadIdx.x] = prm.trig[threadIdx.x];
    __syncthreads();
    const int j = blockIdx.y;
    const int N = prm.N, nh = prm.nh;
    const long long plane = (long long)N * nh;
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= plane) return;
    double2 *Hj = prm.H + (size_t)j * plane;
    if (j >= prm.n_valid) {
        Hj[e] = make_double2(0.0, 0.0);
        if (e == 0) prm.D[j] = make_double2(0.0, 0.0);
        return;
    }
    const PixelRec rec = prm.pix[j];
    const float2 gv = prm.G[prm.goff[j] + e];
    const int iy = (int)(e / nh), ix = (int)(e - (long long)iy * nh);
    if (e == 0) prm.D[j] = make_double2(rec.sw * (double)gv.x, rec.sw * (double)gv.y);
    if (e == 0 || iy == N / 2 || ix == N / 2) {
        Hj[e] = make_double2(0.0, 0.0);
        return;
    }
    double ctop[CHI_DEG + 1];
    chi_tops(prm.op.chi_c, ctop);
    Hj[e] = corrected_value(prm, T, ctop, rec, gv, iy, ix);
}

// ---------------------------------------------------------------------------
// loss path, fused form for power-of-two N <= 1024: the inverse real 2D
// transform split into a column pass (complex, along iy, for each stored
// column ix) that computes the corrected values itself, and a row pass (the
// real transform of each row's half spectrum) that goes straight on to the
// phases and their moments; neither the corrected planes nor the real images
// make a round trip through HBM.  Both passes run self-sorting (Stockham)
// transforms in LDS, radix 8 in registers (one radix-4 or radix-2 pass first
// when log2 N is not a multiple of 3), with the twiddles e^{+2 pi i m / N},
// m < N/2, from a host table in long double.
// ---------------------------------------------------------------------------
constexpr int LOSS_E = 2048;                     // complex values a block transforms at once
constexpr int LOSS_EP = LOSS_E + LOSS_E / 8;     // the same, padded (loss_pad)

// LDS slot of sequence element i: one spare slot per 8, so the first pass's
// stride-8 stores of a wave's lanes fall in distinct banks
__device__ __forceinline__ int loss_pad(int i) { return i + (i >> 3); }

__device__ __forceinline__ double2 c_mul(double2 a, double2 b) {
    return make_double2(fma(a.x, b.x, -(a.y * b.y)), fma(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ double2 c_add(double2 a, double2 b) { return make_double2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ double2 c_sub(double2 a, double2 b) { return make_double2(a.x - b.x, a.y - b.y); }

// In-register DFT of length R in {2, 4, 8} with e^{+2 pi i r k / R}; the
// length-8 one from two length-4 ones (even and odd r) and the factors
// e^{i pi k / 4}.
template <int R>
__device__ __forceinline__ void dft_small(double2 (&v)[R]) {
    if constexpr (R == 2) {
        const double2 t = v[0];
        v[0] = c_add(t, v[1]);
        v[1] = c_sub(t, v[1]);
    } else if constexpr (R == 4) {
        const double2 a = c_add(v[0], v[2]), b = c_sub(v[0], v[2]);
        const double2 c = c_add(v[1], v[3]), d = c_sub(v[1], v[3]);
        const double2 id = make_double2(-d.y, d.x);   // i d
        v[0] = c_add(a, c);
        v[1] = c_add(b, id);
        v[2] = c_sub(a, c);
        v[3] = c_sub(b, id);
    } else {
        double2 e[4] = {v[0], v[2], v[4], v[6]};
        double2 o[4] = {v[1], v[3], v[5], v[7]};
        dft_small<4>(e);
        dft_small<4>(o);
        const double h = 0.70710678118654752440;   // 1 / sqrt 2
        const double2 t1 = make_double2((o[1].x - o[1].y) * h, (o[1].x + o[1].y) * h);    // e^{i pi/4} o1
        const double2 t2 = make_double2(-o[2].y, o[2].x);                                // i o2
        const double2 t3 = make_double2(-(o[3].x + o[3].y) * h, (o[3].x - o[3].y) * h);  // e^{3 i pi/4} o3
        v[0] = c_add(e[0], o[0]);
        v[4] = c_sub(e[0], o[0]);
        v[1] = c_add(e[1], t1);
        v[5] = c_sub(e[1], t1);
        v[2] = c_add(e[2], t2);
        v[6] = c_sub(e[2], t2);
        v[3] = c_add(e[3], t3);
        v[7] = c_sub(e[3], t3);
    }
}

// One Stockham pass of radix R over nt length-N sequences (sequence t at
// elements t N .. t N + N - 1, slots loss_pad of those): sub-transforms of
// length Ns are done; butterfly j of a sequence reads elements j + r N/R,
// applies e^{+2 pi i k r / (Ns R)} (k = j mod Ns) and writes its R outputs
// to (j - k) R + k + r Ns.  A 256-thread block holds at most LOSS_E values,
// so a thread has 8 / R butterflies; all are read before the barrier and
// written after it (in place).
template <int R>
__device__ __forceinline__ void stockham_pass(double2 *A, int nt, int N, int logN, int Ns, const double2 *tw) {
    constexpr int BPT = 8 / R;
    const int NR = N / R;
    const int lognr = logN - (R == 8 ? 3 : (R == 4 ? 2 : 1));
    const int nbut = nt * NR;
    const int step = N / (Ns * R);   // twiddle index per unit of k r
    double2 v[BPT][R];
    int obase[BPT];
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
        const int b = threadIdx.x + u * 256;
        obase[u] = -1;
        if (b < nbut) {
            const int c = b >> lognr, j = b - (c << lognr);
            const int k = j & (Ns - 1);
#pragma unroll
            for (int r = 0; r < R; ++r) v[u][r] = A[loss_pad(c * N + j + r * NR)];
#pragma unroll
            for (int r = 1; r < R; ++r) {
                const int idx = k * r * step;   // < N
                double2 w;
                if (idx < (N >> 1)) {
                    w = tw[idx];
                } else {
                    w = tw[idx - (N >> 1)];
                    w.x = -w.x;
                    w.y = -w.y;
                }
                v[u][r] = c_mul(v[u][r], w);
            }
            obase[u] = c * N + (j - k) * R + k;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
        if (obase[u] < 0) continue;
        dft_small<R>(v[u]);
#pragma unroll
        for (int r = 0; r < R; ++r) A[loss_pad(obase[u] + r * Ns)] = v[u][r];
    }
    __syncthreads();
}

// Unnormalized inverse DFT of nt length-N sequences in place (natural order
// in and out); nt N <= LOSS_E.  Every thread of the 256-thread block calls it
// after the input is in LDS and visible (a barrier).
__device__ __forceinline__ void fft_inverse_stockham(double2 *A, int nt, int N, int logN, const double2 *tw) {
    int Ns = 1;
    const int lead = logN % 3;
    if (lead == 1) {
        stockham_pass<2>(A, nt, N, logN, Ns, tw);
        Ns = 2;
    } else if (lead == 2) {
        stockham_pass<4>(A, nt, N, logN, Ns, tw);
        Ns = 4;
    }
    for (; Ns < N; Ns *= 8) stockham_pass<8>(A, nt, N, logN, Ns, tw);
}

// Item (column block, pixel j of the chunk): columns ix0 .. ix0 + cw - 1 of
// H_j over all N rows, transformed along iy: Y_j(y, ix) = sum_iy H_j(iy, ix)
// e^{+2 pi i iy y / N}.  The item at ix0 = 0 also writes D_j.
// The n_items = ncb cn items are spread over a grid of 8 m blocks that loop:
// block b takes virtual items v = b, b + grid, ...  Workgroups go to the 8
// XCDs in turn, so v maps to item (v mod 8) per + v/8 (per = n_items / 8;
// the last n_items mod 8 map to themselves): each XCD runs a contiguous
// stretch of items, and the column blocks that share G's 128-byte lines meet
// them in that XCD's L2.  A block loads the next item's G values while it
// transforms the current one.
struct LossColItem {
    int j, ix0;
};

__device__ __forceinline__ LossColItem loss_col_item(int v, int per, int ncb, int cw) {
    const int item = v < (per << 3) ? (v & 7) * per + (v >> 3) : v;
    LossColItem it;
    it.j = item / ncb;
    it.ix0 = (item - it.j * ncb) * cw;
    return it;
}

__global__ __launch_bounds__(256, 3) void loss_column_kernel(CorrParams prm, const double2 *tw, int logN, int cw,
                                                             int ncb, int n_items) {
    extern __shared__ double2 lds[];
    double2 *T = lds;                         // [TRIG_N]
    double2 *W = T + TRIG_N;                  // [N/2]
    double2 *A = W + (prm.N >> 1);            // [LOSS_EP]: cw columns of N, padded
    const int N = prm.N, nh = prm.nh;
    for (int i = threadIdx.x; i < TRIG_N; i += blockDim.x) T[i] = prm.trig[i];
    for (int i = threadIdx.x; i < (N >> 1); i += blockDim.x) W[i] = tw[i];
    double ctop[CHI_DEG + 1];
    chi_tops(prm.op.chi_c, ctop);
    // element e = iy cw + c, the thread's elements e = tid + 256 s; with cw a
    // power of two (N >= 64) its column c stays fixed, with no division
    constexpr int EPT = LOSS_E / 256;
    const int n = N * cw;
    const bool pow2 = (cw & (cw - 1)) == 0;
    const int lc = pow2 ? __ffs(cw) - 1 : 0;
    // (row, column) of the thread's element s
    auto rc = [&](int s, int &iy, int &c) {
        const int e = (int)threadIdx.x + 256 * s;
        if (pow2) {
            iy = e >> lc;
            c = e & (cw - 1);
        } else {
            iy = e / cw;
            c = e - iy * cw;
        }
    };
    const int per = n_items >> 3;
    const int stride = gridDim.x;
    int v = blockIdx.x;
    if (v >= n_items) return;
    // the first item's G values
    LossColItem it = loss_col_item(v, per, ncb, cw);
    float2 gv[EPT];
    {
        const float2 *Gj = prm.G + prm.goff[it.j];
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int e = threadIdx.x + 256 * s;
            int iy, c;
            rc(s, iy, c);
            gv[s] = make_float2(0.0f, 0.0f);
            if (e < n && it.ix0 + c < nh) gv[s] = Gj[(size_t)iy * nh + it.ix0 + c];
        }
    }
    while (true) {
        const int j = it.j, ix0 = it.ix0;
        const PixelRec rec = prm.pix[j];
        if (ix0 == 0 && threadIdx.x == 0) {
            const float2 g0 = prm.G[prm.goff[j]];
            prm.D[j] = make_double2(rec.sw * (double)g0.x, rec.sw * (double)g0.y);
        }
        __syncthreads();   // tables loaded; the previous item's transform is read
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int e = threadIdx.x + 256 * s;
            if (e >= n) continue;
            int iy, c;
            rc(s, iy, c);
            const int ix = ix0 + c;
            double2 h = make_double2(0.0, 0.0);
            if (ix < nh && !(iy == 0 && ix == 0) && iy != N / 2 && ix != N / 2)
                h = corrected_value(prm, T, ctop, rec, gv[s], iy, ix);
            A[loss_pad(c * N + iy)] = h;
        }
        // the next item's G values go out before this item's transform
        const int vn = v + stride;
        LossColItem nx = it;
        if (vn < n_items) {
            nx = loss_col_item(vn, per, ncb, cw);
            const float2 *Gn = prm.G + prm.goff[nx.j];
#pragma unroll
            for (int s = 0; s < EPT; ++s) {
                const int e = threadIdx.x + 256 * s;
                int iy, c;
                rc(s, iy, c);
                gv[s] = make_float2(0.0f, 0.0f);
                if (e < n && nx.ix0 + c < nh) gv[s] = Gn[(size_t)iy * nh + nx.ix0 + c];
            }
        }
        __syncthreads();
        fft_inverse_stockham(A, cw, N, logN, W);
        double2 *Yj = prm.H + (size_t)j * N * nh;
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int e = threadIdx.x + 256 * s;
            int y, c;
            rc(s, y, c);
            const int ix = ix0 + c;
            if (e < n && ix < nh) Yj[(size_t)y * nh + ix] = A[loss_pad(c * N + y)];
        }
        if (vn >= n_items) break;
        v = vn;
        it = nx;
    }
}

// Block (row pair p, pixel group g): rows p and p + N/2 of every pixel j = g,
// g + ng, ... of the chunk, LOSS_E / N pixels at a time.  The two rows' half
// spectra, each extended by X(N - kx) = conj X(kx), go into one complex
// transform as a + i b (both images are real), so its real part is row p's
// image and its imaginary part row p + N/2's.  theta = atan2(img + Im D_j,
// Re D_j); each thread adds w_j theta and w_j theta^2 for its positions over
// the group's pixels in order and writes them to the group's partial planes.
// MAXP = max(1, N / 256) positions per thread and row.
template <int MAXP>
__global__ __launch_bounds__(256, (MAXP >= 4 ? 2 : 3)) void loss_row_kernel(const double2 *Y, const double2 *D, const PixelBase *pb,
                                                       int cn, int N, int nh, const double2 *tw, int logN, int ng,
                                                       const double *atab, double *s1p, double *s2p) {
    extern __shared__ double2 lds[];
    double2 *W = lds;              // [N/2]
    double2 *Z = W + (N >> 1);     // [LOSS_EP]: P transforms of N, padded
    double *AT = (double *)(Z + LOSS_EP);   // [ATAN_N] atan(i/64)
    for (int i = threadIdx.x; i < (N >> 1); i += blockDim.x) W[i] = tw[i];
    for (int i = threadIdx.x; i < ATAN_N; i += blockDim.x) AT[i] = atab[i];
    const int p = blockIdx.x, g = blockIdx.y;
    const int ya = p, yb = p + (N >> 1);
    const int P = LOSS_E >> logN;            // pixels per batch
    const int npx = (cn - g + ng - 1) / ng;  // the group's pixels g + ng m, m < npx
    double a1[2 * MAXP], a2[2 * MAXP];
#pragma unroll
    for (int m = 0; m < 2 * MAXP; ++m) a1[m] = a2[m] = 0.0;
    const size_t plane = (size_t)N * nh;
    for (int m0 = 0; m0 < npx; m0 += P) {
        const int nb = (npx - m0) < P ? (npx - m0) : P;
        // the batch's row values, all loaded before the first is used
        constexpr int EPT = LOSS_E / 256;
        double2 va[EPT], vb[EPT];
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int e = threadIdx.x + 256 * s;
            va[s] = vb[s] = make_double2(0.0, 0.0);
            if (e < (nb << logN)) {
                const int t = e >> logN, kx = e & (N - 1);
                const size_t jo = (size_t)(g + ng * (m0 + t)) * plane;
                const int kk = kx <= (N >> 1) ? kx : N - kx;
                va[s] = Y[jo + (size_t)ya * nh + kk];
                vb[s] = Y[jo + (size_t)yb * nh + kk];
            }
        }
        __syncthreads();   // the previous batch's transforms are read
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int e = threadIdx.x + 256 * s;
            if (e < (nb << logN)) {
                double2 a = va[s], b = vb[s];
                if ((e & (N - 1)) > (N >> 1)) {
                    a.y = -a.y;
                    b.y = -b.y;
                }
                Z[loss_pad(e)] = make_double2(a.x - b.y, a.y + b.x);
            }
        }
        __syncthreads();
        fft_inverse_stockham(Z, nb, N, logN, W);
        for (int t = 0; t < nb; ++t) {
            const int j = g + ng * (m0 + t);
            const double2 d = D[j];
            const double w = pb[j].w;
            const bool x0 = d.x == 0.0;   // atan2(y, 0): the library's (uniform per pixel)
            const double rx = x0 ? 0.0 : 1.0 / d.x;
#pragma unroll
            for (int m = 0; m < MAXP; ++m) {
                const int x = threadIdx.x + m * 256;
                if (x < N) {
                    const double2 z = Z[loss_pad((t << logN) + x)];
                    double ta, tb;
                    if (x0) {
                        ta = atan2(z.x + d.y, d.x);
                        tb = atan2(z.y + d.y, d.x);
                    } else {
                        ta = atan2_tab(z.x + d.y, d.x, rx, AT);
                        tb = atan2_tab(z.y + d.y, d.x, rx, AT);
                    }
                    a1[m] = fma(w, ta, a1[m]);
                    a2[m] = fma(w * ta, ta, a2[m]);
                    a1[MAXP + m] = fma(w, tb, a1[MAXP + m]);
                    a2[MAXP + m] = fma(w * tb, tb, a2[MAXP + m]);
                }
            }
        }
    }
    const size_t nn = (size_t)N * N;
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
        const int x = threadIdx.x + m * 256;
        if (x < N) {
            s1p[(size_t)g * nn + (size_t)ya * N + x] = a1[m];
            s2p[(size_t)g * nn + (size_t)ya * N + x] = a2[m];
            s1p[(size_t)g * nn + (size_t)yb * N + x] = a1[MAXP + m];
            s2p[(size_t)g * nn + (size_t)yb * N + x] = a2[MAXP + m];
        }
    }
}

// s1 += the groups' partials, in group order (deterministic)
__global__ __launch_bounds__(256) void loss_groups_kernel(const double *s1p, const double *s2p, int ng, long long nn,
                                                          double *s1, double *s2) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long r = (long long)blockIdx.x * blockDim.x + threadIdx.x; r < nn; r += stride) {
        double a = s1[r], b = s2[r];
        for (int g = 0; g < ng; ++g) {
            a += s1p[(size_t)g * nn + r];
            b += s2p[(size_t)g * nn + r];
        }
        s1[r] = a;
        s2[r] = b;
    }
}

// r over the N^2 scan positions: theta_j = atan2(img_j[r] + Im D_j, Re D_j)
// (img_j the unnormalized inverse real transform of H_j); s1 += w_j theta_j,
// s2 += w_j theta_j^2 over the chunk's pixels in order.
__global__ __launch_bounds__(256) void phase_moments_kernel(const double *img, const double2 *D, const PixelBase *pb,
                                                            int cn, long long nn, double *s1, double *s2) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long r = (long long)blockIdx.x * blockDim.x + threadIdx.x; r < nn; r += stride) {
        double a1 = s1[r], a2 = s2[r];
#pragma unroll 4
        for (int j = 0; j < cn; ++j) {
            const double2 d = D[j];
            const double w = pb[j].w;
            const double th = atan2(img[(size_t)j * nn + r] + d.y, d.x);
            a1 = fma(w, th, a1);
            a2 = fma(w * th, th, a2);
        }
        s1[r] = a1;
        s2[r] = a2;
    }
}

// mean = s1 / W, var = s2 / W - mean^2; block b writes the sum of var over
// its positions (b, b + nblk, ... in 256-wide steps, fixed tree).
__global__ __launch_bounds__(256) void loss_partial_kernel(const double *s1, const double *s2, long long nn, double W,
                                                           double *mean_out, double *part) {
    __shared__ double sh[256];
    const long long stride = (long long)gridDim.x * blockDim.x;
    double acc = 0.0;
    for (long long r = (long long)blockIdx.x * blockDim.x + threadIdx.x; r < nn; r += stride) {
        const double m = s1[r] / W;
        if (mean_out) mean_out[r] = m;
        acc += s2[r] / W - m * m;
    }
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) sh[threadIdx.x] += sh[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = sh[0];
}

// loss = (sum of the blocks' sums, in block order) / nn
__global__ void loss_final_kernel(const double *part, int nblk, long long nn, double *loss) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        double s = 0.0;
        for (int b = 0; b < nblk; ++b) s += part[b];
        loss[0] = s / (double)nn;
    }
}

// Per band tile: the reduced sums -> S, N outputs and the tile's agreement
// partials (|S_b|^2 / N_b and P summed over the lanes by a fixed tree).
template <int MAXB>
__global__ __launch_bounds__(64) void ssb_write_kernel(SsbParams prm, double *tile_part) {
    constexpr int NACC = 3 * MAXB + 1;
    const int lane = threadIdx.x;
    const int t = blockIdx.x;
    const SsbTile *tile = prm.tiles + t;
    const int yh = tile->lyh[lane];
    const int ix = tile->lix[lane];
    const bool valid = (tile->valid >> lane) & 1ull;
    const int iy = yh < 0 ? yh + prm.N : yh;
    const long long lane_off = valid ? (long long)iy * prm.nh + ix : 0;
    const double *pi = prm.partial + (size_t)prm.seg_first[t] * (NACC * 64);
    const size_t plane = (size_t)prm.N * prm.nh;
    double part[MAXB + 1];
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
        const double sr = pi[(3 * b) * 64 + lane], si = pi[(3 * b + 1) * 64 + lane], nn = pi[(3 * b + 2) * 64 + lane];
        const bool ok = valid && b < prm.B;
        if (ok && prm.S_out) prm.S_out[(size_t)b * plane + lane_off] = make_double2(sr, si);
        if (ok && prm.N_out) prm.N_out[(size_t)b * plane + lane_off] = nn;
        part[b] = (ok && nn > 0.0) ? (sr * sr + si * si) / nn : 0.0;
    }
    part[MAXB] = valid ? pi[(NACC - 1) * 64 + lane] : 0.0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
        for (int b = 0; b <= MAXB; ++b) part[b] += __shfl_xor(part[b], off);
    }
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b <= MAXB; ++b) tile_part[(size_t)t * (MAXB + 1) + b] = part[b];
    }
}

__global__ void agreement_kernel(const double *partial, int n_tiles, int stride, int B, double *E) {
    // one block of 64 threads; thread t sums tiles t, t+64, ... then a fixed tree
    __shared__ double sh[64];
    const int t = threadIdx.x;
    for (int b = 0; b <= B; ++b) {
        const int col = (b == B) ? stride - 1 : b;
        double s = 0.0;
        for (int i = t; i < n_tiles; i += 64) s += partial[(size_t)i * stride + col];
        sh[t] = s;
        __syncthreads();
        for (int h = 32; h >= 1; h >>= 1) {
            if (t < h) sh[t] += sh[t + h];
            __syncthreads();
        }
        if (t == 0) E[b] = sh[0];
        __syncthreads();
    }
    if (t == 0) {
        const double den = E[B];
        for (int b = 0; b < B; ++b) E[b] = E[b] / den;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

#define DSP_CHECK_LAUNCH() \
    do { hipError_t e_ = hipGetLastError(); if (e_ != hipSuccess) return e_; } while (0)

hipError_t launch_pixel_terms(const PixelBase *in, PixelRec *out, int n_pix, const ApertureDev &ap, const OpticsDev &op,
                              double *chi_tab, int chi_stride, double *tay, hipStream_t st) {
    if (n_pix <= 0) return hipSuccess;
    pixel_terms_kernel<<<(n_pix + 255) / 256, 256, 0, st>>>(in, out, n_pix, ap, op, chi_tab, chi_stride, tay);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

// Calls F<NJ, METHOD>::run(args...) for the compiled (slots, method) pairs.
template <template <int, int> class F, class... Args>
static hipError_t gram_dispatch(int nj, int method, Args &&...args) {
    if (method == 0) {
        switch (nj) {
            case 1: return F<1, 0>::run(args...);
            case 2: return F<2, 0>::run(args...);
            case 3: return F<3, 0>::run(args...);
            case 4: return F<4, 0>::run(args...);
            case 5: return F<5, 0>::run(args...);
            case 6: return F<6, 0>::run(args...);
            case 7: return F<7, 0>::run(args...);
            case 8: return F<8, 0>::run(args...);
            default: return hipErrorInvalidValue;
        }
    }
    if (method == 2) {
        switch (nj) {
            case 1: return F<1, 2>::run(args...);
            case 2: return F<2, 2>::run(args...);
            case 3: return F<3, 2>::run(args...);
            case 4: return F<4, 2>::run(args...);
            case 5: return F<5, 2>::run(args...);
            case 6: return F<6, 2>::run(args...);
            case 7: return F<7, 2>::run(args...);
            case 8: return F<8, 2>::run(args...);
            case 9: return F<9, 2>::run(args...);
            default: return hipErrorInvalidValue;
        }
    }
    switch (nj) {
        case 1: return F<1, 1>::run(args...);
        case 2: return F<2, 1>::run(args...);
        case 3: return F<3, 1>::run(args...);
        case 4: return F<4, 1>::run(args...);
        case 5: return F<5, 1>::run(args...);
        case 6: return F<6, 1>::run(args...);
        default: return hipErrorInvalidValue;
    }
}

template <int NJ, int METHOD>
struct GramLaunch {
    static hipError_t run(const GramParams &prm, int n_waves, hipStream_t st) {
        if (prm.op.pt2 != 0.0) gram_kernel<NJ, METHOD, true><<<n_waves, 64, 0, st>>>(prm);
        else gram_kernel<NJ, METHOD, false><<<n_waves, 64, 0, st>>>(prm);
        DSP_CHECK_LAUNCH();
        return hipSuccess;
    }
};

template <int NJ, int METHOD>
struct GramFixupLaunch {
    static hipError_t run(const GramParams &prm, int n_tiles, hipStream_t st) {
        const int nacc = GramShape<NJ, METHOD>::NACC;
        gram_reduce_kernel<<<dim3((nacc + 3) / 4, n_tiles), 256, 0, st>>>(prm, nacc);
        DSP_CHECK_LAUNCH();
        gram_write_kernel<NJ, METHOD><<<n_tiles, 64, 0, st>>>(prm);
        DSP_CHECK_LAUNCH();
        return hipSuccess;
    }
};

template <int NJ, int METHOD>
struct GramOccupancy {
    static hipError_t run(int *blocks_per_cu) {
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, gram_kernel<NJ, METHOD, false>, 64, 0);
    }
};

int gram_nacc(int nj, int method) {
    if (method == 2) return 2 * nj;
    const int nc = method == 0 ? nj : 2 * nj;
    const int d = nc + 1;
    return d + d * (d - 1);
}

hipError_t gram_occupancy(int nj, int method, int *blocks_per_cu) {
    return gram_dispatch<GramOccupancy>(nj, method, blocks_per_cu);
}

hipError_t launch_gram(const GramParams &prm, int nj, int method, int n_waves, hipStream_t st) {
    if (n_waves <= 0) return hipSuccess;
    return gram_dispatch<GramLaunch>(nj, method, prm, n_waves, st);
}

hipError_t launch_gram_fixup(const GramParams &prm, int nj, int method, int n_tiles, hipStream_t st) {
    if (n_tiles <= 0) return hipSuccess;
    return gram_dispatch<GramFixupLaunch>(nj, method, prm, n_tiles, st);
}

hipError_t launch_work_count(const GramParams &prm, int method, int n_tiles, unsigned long long *out,
                             hipStream_t st) {
    if (n_tiles <= 0) return hipSuccess;
    if (method == 0) work_count_kernel<0><<<n_tiles, 64, 0, st>>>(prm, out);
    else work_count_kernel<1><<<n_tiles, 64, 0, st>>>(prm, out);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_phase_from_complex(const double2 *csys, double2 *psys, int a_max, int n_q, hipStream_t st) {
    const long long n = (long long)n_q * tri_size(a_max + 1);
    if (n <= 0) return hipSuccess;
    phase_from_complex_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(csys, psys, a_max, n_q);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_eig(const EigParams &prm, int A, hipStream_t st) {
    if (prm.n <= 0) return hipSuccess;
    const int blocks = (prm.n + 63) / 64;
    switch (A) {
        case 1: eig_kernel<1><<<blocks, 64, 0, st>>>(prm); break;
        case 2: eig_kernel<2><<<blocks, 64, 0, st>>>(prm); break;
        case 3: eig_kernel<3><<<blocks, 64, 0, st>>>(prm); break;
        case 4: eig_kernel<4><<<blocks, 64, 0, st>>>(prm); break;
        case 5: eig_kernel<5><<<blocks, 64, 0, st>>>(prm); break;
        case 6: eig_kernel<6><<<blocks, 64, 0, st>>>(prm); break;
        case 7: eig_kernel<7><<<blocks, 64, 0, st>>>(prm); break;
        case 8: eig_kernel<8><<<blocks, 64, 0, st>>>(prm); break;
        default: return hipErrorInvalidValue;
    }
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_solve(const SolveParams &prm, int A, int method, hipStream_t st) {
    if (prm.n <= 0) return hipSuccess;
    const int blocks = (prm.n + 63) / 64;
    if (A == 0) {
        solve_empty_kernel<<<blocks, 64, 0, st>>>(prm, method == 0 ? 1 : 2);
        DSP_CHECK_LAUNCH();
        return hipSuccess;
    }
    if (method == 0) {
        switch (A) {
            case 1: solve_phase_kernel<1><<<blocks, 64, 0, st>>>(prm); break;
            case 2: solve_phase_kernel<2><<<blocks, 64, 0, st>>>(prm); break;
            case 3: solve_phase_kernel<3><<<blocks, 64, 0, st>>>(prm); break;
            case 4: solve_phase_kernel<4><<<blocks, 64, 0, st>>>(prm); break;
            case 5: solve_phase_kernel<5><<<blocks, 64, 0, st>>>(prm); break;
            case 6: solve_phase_kernel<6><<<blocks, 64, 0, st>>>(prm); break;
            case 7: solve_phase_kernel<7><<<blocks, 64, 0, st>>>(prm); break;
            case 8: solve_phase_kernel<8><<<blocks, 64, 0, st>>>(prm); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (A) {
            case 1: solve_complex_kernel<1><<<blocks, 64, 0, st>>>(prm); break;
            case 2: solve_complex_kernel<2><<<blocks, 64, 0, st>>>(prm); break;
            case 3: solve_complex_kernel<3><<<blocks, 64, 0, st>>>(prm); break;
            case 4: solve_complex_kernel<4><<<blocks, 64, 0, st>>>(prm); break;
            case 5: solve_complex_kernel<5><<<blocks, 64, 0, st>>>(prm); break;
            case 6:   // factor in LDS: SOLVE_LDS_THREADS threads per block
                static_assert(SolveInLds<6>::value, "the six-alias factor lives in LDS");
                solve_complex_kernel<6><<<(prm.n + SOLVE_LDS_THREADS - 1) / SOLVE_LDS_THREADS, SOLVE_LDS_THREADS,
                                          0, st>>>(prm);
                break;
            default: return hipErrorInvalidValue;
        }
    }
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_fill_zero(double *p, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    fill_zero_kernel<<<(unsigned)blocks, 256, 0, st>>>(p, n);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_scatter(const ScatterParams &prm, hipStream_t st) {
    const size_t total = (size_t)prm.SC * prm.n_q;
    if (total == 0) return hipSuccess;
    scatter_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(prm);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_export(const double2 *sys, int n_q, int D, double2 *dense, hipStream_t st) {
    const size_t total = (size_t)n_q * D * D;
    if (total == 0) return hipSuccess;
    export_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(sys, n_q, D, dense);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

int ssb_maxb(int B) { return B <= 1 ? 1 : (B <= 2 ? 2 : (B <= 4 ? 4 : 8)); }

int ssb_nacc(int maxb) { return 3 * maxb + 1; }

hipError_t ssb_occupancy(int maxb, int *blocks_per_cu) {
    switch (maxb) {
        case 1: return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, ssb_kernel<1, false, 0>, 64, 0);
        case 2: return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, ssb_kernel<2, false, 0>, 64, 0);
        case 4: return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, ssb_kernel<4, false, 0>, 64, 0);
        case 8: return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, ssb_kernel<8, false, 0>, 64, 0);
        default: return hipErrorInvalidValue;
    }
}

template <int MAXB, bool DEPTH>
static void ssb_dispatch_h(const SsbParams &prm, int h16, int n_waves, hipStream_t st) {
    if (h16 == 2) ssb_kernel<MAXB, DEPTH, 2><<<n_waves, 64, 0, st>>>(prm);
    else if (h16 == 1) ssb_kernel<MAXB, DEPTH, 1><<<n_waves, 64, 0, st>>>(prm);
    else ssb_kernel<MAXB, DEPTH, 0><<<n_waves, 64, 0, st>>>(prm);
}

template <int MAXB>
static void ssb_dispatch(const SsbParams &prm, bool depth, int h16, int n_waves, hipStream_t st) {
    if (depth) ssb_dispatch_h<MAXB, true>(prm, h16, n_waves, st);
    else ssb_dispatch_h<MAXB, false>(prm, h16, n_waves, st);
}

hipError_t launch_herm16(const float2 *G, int n_bf, int N, int nh, bool rows, short2 *Q, float *scale,
                         hipStream_t st) {
    const long long plane = (long long)N * nh;
    if (n_bf <= 0 || plane <= 0) return hipSuccess;
    if (rows && nh <= 64 * HERM16_RPL) {
        const long long n_rows = (long long)n_bf * N;
        herm16_rows_fused_kernel<<<(unsigned)((n_rows + 3) / 4), 256, 0, st>>>(G, n_rows, nh, scale, Q);
        DSP_CHECK_LAUNCH();
        return hipSuccess;
    }
    if (rows) {
        const long long n_rows = (long long)n_bf * N;
        herm16_row_scale_kernel<<<(unsigned)((n_rows + 3) / 4), 256, 0, st>>>(G, n_rows, nh, scale);
    } else {
        herm16_scale_kernel<<<n_bf, 256, 0, st>>>(G, plane, scale);
    }
    DSP_CHECK_LAUNCH();
    // pairs per plane over blocks of 256 threads, about 8 pairs per thread
    // (two per step)
    const long long npair = plane / 2;
    const unsigned bx = (unsigned)std::max<long long>(1, std::min<long long>((npair + 2047) / 2048, 4096));
    const dim3 grid(bx, (unsigned)std::min(n_bf, 65535));
    if (rows) herm16_pack_kernel<true><<<grid, 256, 0, st>>>(G, plane, N, nh, n_bf, scale, Q);
    else herm16_pack_kernel<false><<<grid, 256, 0, st>>>(G, plane, N, nh, n_bf, scale, Q);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

static unsigned grid_blocks(long long n) {
    const long long b = (n + 255) / 256;
    return (unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

hipError_t launch_preview_dc(const PixelBase *pix, const long long *goff, int n_pix, const float2 *G, double2 *dc,
                             hipStream_t st) {
    preview_dc_kernel<<<1, 256, 0, st>>>(pix, goff, n_pix, G, dc);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_preview_spectrum(const double2 *S, const double2 *dc, long long n, double2 *P, hipStream_t st) {
    preview_spectrum_kernel<<<grid_blocks(n), 256, 0, st>>>(S, dc, n, P);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_preview_phase(double *img, long long n, const double2 *dc, hipStream_t st) {
    preview_phase_kernel<<<grid_blocks(n), 256, 0, st>>>(img, n, dc);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_corrected_half(const CorrParams &prm, int n_planes, hipStream_t st) {
    const long long plane = (long long)prm.N * prm.nh;
    corrected_half_kernel<<<dim3((unsigned)((plane + 255) / 256), (unsigned)n_planes), 256, 0, st>>>(prm);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

int loss_fused_cols(int N) { return std::max(1, std::min(LOSS_E / N, N / 2 + 1)); }

hipError_t launch_loss_fused(const CorrParams &prm, const double2 *tw, const double *atab, int cn, const PixelBase *pb,
                             int ng, double *s1p, double *s2p, double *s1, double *s2, hipStream_t st) {
    const int N = prm.N, nh = prm.nh;
    int logN = 0;
    while ((1 << logN) < N) ++logN;
    if ((1 << logN) != N || N < 8 || N > 1024 || cn <= 0 || ng <= 0) return hipErrorInvalidValue;
    const int cw = loss_fused_cols(N);
    const size_t lds_a = (size_t)(TRIG_N + N / 2 + LOSS_EP) * sizeof(double2);
    // looping blocks: about eight items each, a multiple of 8 blocks (XCDs)
    const int ncb = (nh + cw - 1) / cw, n_items = ncb * cn;
    const int grid_a = std::max(8, (n_items / 8 + 7) / 8 * 8);
    loss_column_kernel<<<(unsigned)grid_a, 256, lds_a, st>>>(prm, tw, logN, cw, ncb, n_items);
    DSP_CHECK_LAUNCH();
    const size_t lds_b = (size_t)(N / 2 + LOSS_EP) * sizeof(double2) + ATAN_N * sizeof(double);
    const dim3 grid_b((unsigned)(N / 2), (unsigned)ng);
    if (N <= 256)
        loss_row_kernel<1><<<grid_b, 256, lds_b, st>>>(prm.H, prm.D, pb, cn, N, nh, tw, logN, ng, atab, s1p, s2p);
    else if (N == 512)
        loss_row_kernel<2><<<grid_b, 256, lds_b, st>>>(prm.H, prm.D, pb, cn, N, nh, tw, logN, ng, atab, s1p, s2p);
    else
        loss_row_kernel<4><<<grid_b, 256, lds_b, st>>>(prm.H, prm.D, pb, cn, N, nh, tw, logN, ng, atab, s1p, s2p);
    DSP_CHECK_LAUNCH();
    const long long nn = (long long)N * N;
    loss_groups_kernel<<<grid_blocks(nn), 256, 0, st>>>(s1p, s2p, ng, nn, s1, s2);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_phase_moments(const double *img, const double2 *D, const PixelBase *pb, int cn, long long nn,
                                double *s1, double *s2, hipStream_t st) {
    phase_moments_kernel<<<grid_blocks(nn), 256, 0, st>>>(img, D, pb, cn, nn, s1, s2);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

int loss_blocks(long long nn) { return (int)std::min<long long>(1024, std::max<long long>(1, (nn + 255) / 256)); }

hipError_t launch_loss(const double *s1, const double *s2, long long nn, double W, double *mean_out, double *part,
                       double *loss, hipStream_t st) {
    const int nb = loss_blocks(nn);
    loss_partial_kernel<<<nb, 256, 0, st>>>(s1, s2, nn, W, mean_out, part);
    DSP_CHECK_LAUNCH();
    loss_final_kernel<<<1, 64, 0, st>>>(part, nb, nn, loss);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

hipError_t launch_ssb(const SsbParams &prm, int n_waves, int n_tiles, double *tile_part, hipStream_t st) {
    if (n_waves <= 0 || n_tiles <= 0) return hipSuccess;
    const int maxb = ssb_maxb(prm.B);
    const int nacc = ssb_nacc(maxb);
    bool depth = false;   // depth terms when any set has a depth
    for (int b = 0; b < prm.B; ++b) depth = depth || prm.pt2[b] != 0.0;
    const int h16 = prm.GQ == nullptr ? 0 : (prm.h16_rows ? 2 : 1);
    switch (maxb) {
        case 1: ssb_dispatch<1>(prm, depth, h16, n_waves, st); break;
        case 2: ssb_dispatch<2>(prm, depth, h16, n_waves, st); break;
        case 4: ssb_dispatch<4>(prm, depth, h16, n_waves, st); break;
        default: ssb_dispatch<8>(prm, depth, h16, n_waves, st); break;
    }
    DSP_CHECK_LAUNCH();
    // reduce each tile's segments (same reduction as the Gram fixup)
    GramParams gp;
    memset(&gp, 0, sizeof gp);
    gp.seg_first = prm.seg_first;
    gp.partial = prm.partial;
    gram_reduce_kernel<<<dim3((nacc + 3) / 4, n_tiles), 256, 0, st>>>(gp, nacc);
    DSP_CHECK_LAUNCH();
    switch (maxb) {
        case 1: ssb_write_kernel<1><<<n_tiles, 64, 0, st>>>(prm, tile_part); break;
        case 2: ssb_write_kernel<2><<<n_tiles, 64, 0, st>>>(prm, tile_part); break;
        case 4: ssb_write_kernel<4><<<n_tiles, 64, 0, st>>>(prm, tile_part); break;
        default: ssb_write_kernel<8><<<n_tiles, 64, 0, st>>>(prm, tile_part); break;
    }
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

int ssb_partial_stride(int B) { return ssb_maxb(B) + 1; }

// ---------------------------------------------------------------------------
// fixed scratch of the allocation-free SSB pass
// ---------------------------------------------------------------------------
// One array per device, part of the library's code object: each GPU the
// library runs on holds its own copy at its own address until the process
// ends.  In host code the name `scratch` is only a host-side stand-in, never
// a device address: host code uses the pointer hipGetSymbolAddress returns
// for the current device (kept per device below), in kernel arguments and
// copies alike.
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(char **out) {
    static std::mutex mu;
    static char *ptrs[64] = {nullptr};
    *out = nullptr;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return e;
    if (device < 0 || device >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[device]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // the current device's copy
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[device] = (char *)p;
    }
    *out = ptrs[device];
    return hipSuccess;
}

hipError_t launch_agreement(const double *partial, int n_tiles, int B, double *E, hipStream_t st) {
    agreement_kernel<<<1, 64, 0, st>>>(partial, n_tiles, ssb_partial_stride(B), B, E);
    DSP_CHECK_LAUNCH();
    return hipSuccess;
}

}  // namespace dsp
