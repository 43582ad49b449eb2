// Internal types shared by the host side (dsp_api.cpp) and the HIP kernels
// (dsp_kernels.hip) of libdsp.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsp {

// ---------------------------------------------------------------------------
// aberration phase as a bivariate polynomial in theta = lambda k + tau
// ---------------------------------------------------------------------------
// chi(theta) = sum_{i + j <= 6} c(i, j) theta_x^i theta_y^j.  A Krivanek term
// t^(n+1) cos(m (p - phi)) equals Re[exp(-i m phi) w^m] (w w*)^((n+1-m)/2) with
// w = theta_x + i theta_y, a homogeneous polynomial of degree n + 1 <= 6.
// Storage: for j = 0..6, coefficients i = 0..6-j contiguous (28 doubles).
constexpr int CHI_DEG = 6;
constexpr int CHI_NCOEF = 28;

__host__ __device__ constexpr int chi_off(int j) { return j * (2 * CHI_DEG + 3 - j) / 2; }

// Horner in theta_x inside Horner in theta_y: 27 FMAs.  top[j] is row j's
// leading coefficient, c[chi_off(j) + 6 - j] (chi_poly passes c's own; the
// Gram kernels pass copies held in vector registers, so that no row's first
// FMA has two scalar operands).
__host__ __device__ inline double chi_poly_top(const double *__restrict__ c, const double *__restrict__ top,
                                               double tx, double ty) {
    double acc = top[6];
#pragma unroll
    for (int j = 5; j >= 0; --j) {
        const double *cj = c + chi_off(j);
        double h = top[j];
#pragma unroll
        for (int i = 5 - j; i >= 0; --i) h = fma(h, tx, cj[i]);
        acc = fma(acc, ty, h);
    }
    return acc;
}

__host__ __device__ inline double chi_poly(const double *__restrict__ c, double tx, double ty) {
    double top[CHI_DEG + 1];
#pragma unroll
    for (int j = 0; j <= CHI_DEG; ++j) top[j] = c[chi_off(j) + CHI_DEG - j];
    return chi_poly_top(c, top, tx, ty);
}

// ---------------------------------------------------------------------------
// chi about a pixel's theta: both lobes' phases from one evaluation
// ---------------------------------------------------------------------------
// The transfer's two lobes at scan frequency Q need chi at theta -/+ d with
// d = lambda Q.  Expanded about theta, chi(theta + d) - chi(theta) =
// E(d) + O(d) with E the terms of even and O those of odd total degree in
// d, so chi(theta - d) - chi(theta) = E - O: one evaluation of E and O
// serves both lobes.  The coefficients t_ab of d_x^a d_y^b come from chi's
// own by a Taylor shift (repeated synthetic division, the Ruffini-Horner
// scheme) in x, then in y: 112 FMAs per theta.  Degree 6 is shift-invariant
// (chi's own coefficients); degrees 1..5 (20 values) depend on theta.
// Per-theta layout (groups as the evaluation reads them):
//   A: t20 t02 t40 t22 t04 | B: t11 t31 t13 |
//   C: t10 t30 t12 t50 t32 t14 | D: t01 t21 t03 t41 t23 t05
constexpr int TAY_N = 20;

__host__ __device__ inline void chi_taylor(const double *__restrict__ c, double tx, double ty,
                                           double *__restrict__ t) {
    double a[CHI_NCOEF];
#pragma unroll
    for (int i = 0; i < CHI_NCOEF; ++i) a[i] = c[i];
    // shift in x: row j is a polynomial of degree 6 - j in theta_x
#pragma unroll
    for (int j = 0; j < CHI_DEG; ++j) {
        const int n = CHI_DEG - j, o = chi_off(j);
#pragma unroll
        for (int k = 0; k < n; ++k)
#pragma unroll
            for (int i = n - 1; i >= k; --i) a[o + i] = fma(tx, a[o + i + 1], a[o + i]);
    }
    // shift in y: column i is a polynomial of degree 6 - i in theta_y
#pragma unroll
    for (int i = 0; i < CHI_DEG; ++i) {
        const int n = CHI_DEG - i;
#pragma unroll
        for (int k = 0; k < n; ++k)
#pragma unroll
            for (int j = n - 1; j >= k; --j) a[chi_off(j) + i] = fma(ty, a[chi_off(j + 1) + i], a[chi_off(j) + i]);
    }
#define DSP_T(x, y) a[chi_off(y) + (x)]
    t[0] = DSP_T(2, 0);  t[1] = DSP_T(0, 2);  t[2] = DSP_T(4, 0);  t[3] = DSP_T(2, 2);  t[4] = DSP_T(0, 4);
    t[5] = DSP_T(1, 1);  t[6] = DSP_T(3, 1);  t[7] = DSP_T(1, 3);
    t[8] = DSP_T(1, 0);  t[9] = DSP_T(3, 0);  t[10] = DSP_T(1, 2); t[11] = DSP_T(5, 0); t[12] = DSP_T(3, 2);
    t[13] = DSP_T(1, 4);
    t[14] = DSP_T(0, 1); t[15] = DSP_T(2, 1); t[16] = DSP_T(0, 3); t[17] = DSP_T(4, 1); t[18] = DSP_T(2, 3);
    t[19] = DSP_T(0, 5);
#undef DSP_T
}

// E(d) and O(d) from the per-theta coefficients t and chi's degree-6 ones
// (c), with X = d_x^2, Y = d_y^2, Z = d_x d_y:
//   E = X (t20 + X (t40 + X c60 + Y c42) + Y (t22 + Y c24)) + Y (t02 + Y (t04 + Y c06))
//     + Z (t11 + X (t31 + X c51 + Y c33) + Y (t13 + Y c15))
//   O = d_x (t10 + X (t30 + X t50 + Y t32) + Y (t12 + Y t14))
//     + d_y (t01 + X (t21 + X t41 + Y t23) + Y (t03 + Y t05))
// 30 FP64 operations.
// The even part reads t[0..7], the odd part t[8..19] (to = t + 8).
__host__ __device__ inline double chi_even(const double *__restrict__ t, const double *__restrict__ c, double X,
                                           double Y, double Z) {
    const double c60 = c[chi_off(0) + 6], c42 = c[chi_off(2) + 4], c24 = c[chi_off(4) + 2], c06 = c[chi_off(6)];
    const double c51 = c[chi_off(1) + 5], c33 = c[chi_off(3) + 3], c15 = c[chi_off(5) + 1];
    const double u = fma(Y, c42, fma(X, c60, t[2]));
    const double v = fma(Y, c24, t[3]);
    const double P = fma(Y, v, fma(X, u, t[0]));
    const double R = fma(Y, fma(Y, c06, t[4]), t[1]);
    const double A = fma(X, P, Y * R);
    const double B = fma(Y, fma(Y, c15, t[7]), fma(X, fma(Y, c33, fma(X, c51, t[6])), t[5]));
    return fma(Z, B, A);
}

__host__ __device__ inline double chi_odd(const double *__restrict__ to, double dx, double dy, double X, double Y) {
    const double C = fma(Y, fma(Y, to[5], to[2]), fma(X, fma(Y, to[4], fma(X, to[3], to[1])), to[0]));
    const double D = fma(Y, fma(Y, to[11], to[8]), fma(X, fma(Y, to[10], fma(X, to[9], to[7])), to[6]));
    return fma(dx, C, dy * D);
}

__host__ __device__ inline void chi_even_odd(const double *__restrict__ t, const double *__restrict__ c, double dx,
                                             double dy, double &E, double &O) {
    const double X = dx * dx, Y = dy * dy, Z = dx * dy;
    E = chi_even(t, c, X, Y, Z);
    O = chi_odd(t + 8, dx, dy, X, Y);
}

// ---------------------------------------------------------------------------
// packed upper-triangle index of an n x n matrix, i <= j
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int tri_idx(int i, int j, int n) { return i * (2 * n - i + 1) / 2 + (j - i); }
__host__ __device__ constexpr int tri_size(int n) { return n * (n + 1) / 2; }

// ---------------------------------------------------------------------------
// device tables
// ---------------------------------------------------------------------------
// One active bright-field pixel as given: k (1/A, scan frame) and its weight.
struct PixelBase {
    double ky, kx;     // 1/A, scan frame
    double w, sw;      // weight and sqrt(w)
};

// Per-prepare pixel record.  Lengths are scaled by lambda, so theta =
// lambda (k -/+ Q) + tau is the pixel's theta(k) = lambda k + tau minus or
// plus lambda Q, and the support test of k' = k -/+ Q is |lambda k|^2 +
// |lambda Q|^2 -/+ 2 (lambda k).(lambda Q) against (lambda r)^2.  The kernels
// form theta(k) = lky + tau_y (a separately rounded add, as chi0 was built),
// so at Q = 0 the two phases agree exactly.  The weight enters the Gram
// through sqrt(w): with u = sqrt(w) T and g' = sqrt(w) g, u^H u = T^H W T,
// u^H g' = T^H W g and |g'|^2 = g^H W g, so the update needs no weight
// products.
struct alignas(16) PixelRec {
    double lky, lkx;   // lambda k (rounded products)
    double amp0;       // sqrt(w) a(k)
    double sw;         // sqrt(w)
    double chi0;       // chi(theta(k)), theta(k) = (lky + tau_y, lkx + tau_x)
    double pad;
};

// ---------------------------------------------------------------------------
// FP64 sine and cosine for the transfer's phase factors
// ---------------------------------------------------------------------------
// Table-driven: x = n pi/128 + r with n = rint(128 x / pi) and |r| <= pi/256,
// by one Cody-Waite step (W. J. Cody and W. Waite, "Software Manual for the
// Elementary Functions", 1980) with the constant P1 = double(pi)/128: x - n P1
// is exact in one FMA for |x| < 2^30 (both terms are multiples of 2^-58, or x
// is below 2^-6 and n is 0 or +-1, with x a multiple of 2^-59, and the
// difference is below 2^-6); the constant's own error, 1e-18 per step of
// pi/128, adds at most 4e-17 |x| rad (4e-14 at |x| = 1e3).  Then sin r = r - r^3/6
// (truncation below r^5/120 = 2.4e-12 at |r| = pi/256) and cos r = 1 - r^2/2
// + r^4/24 (below 5e-15), and the angle addition with T[n mod 256] = (cos,
// sin)(n pi/128).  Absolute error about 2.4e-12: a lobe's value moves by that
// fraction of its amplitude, a Gram entry by at most 5e-12 of the system's
// largest and an SSB sum term likewise, within the 1e-9 and 1e-5 bounds.
// Branch-free; T is 256 double2 (4 KB).
constexpr int TRIG_N = 256;

__host__ __device__ inline void sincos_tab(double x, const double2 *__restrict__ T, double &s, double &c) {
    const double n = rint(x * 40.74366543152521);          // 128 / pi
    const double r = fma(-n, 0.02454369260617026, x);      // P1 = pi / 128
    const double z = r * r;
    const double sr = fma(r * z, -1.6666666666666666667e-01, r);
    const double cr = fma(z, fma(z, 4.1666666666666666667e-02, -0.5), 1.0);
    const double2 t = T[((int)n) & (TRIG_N - 1)];
    s = fma(t.y, cr, t.x * sr);
    c = fma(t.x, cr, -(t.y * sr));
}

// ---------------------------------------------------------------------------
// FP64 atan2 of the loss path's phases
// ---------------------------------------------------------------------------
// theta = atan2(y, x) where x (a pixel's Re D) is the same at every scan
// position, so t = y (1/x) with 1/x formed once per pixel.  |t| > 1 folds by
// atan |t| = pi/2 - atan(1/|t|); u in [0, 1] is reduced against c = i/64, i =
// rint(64 u), by atan u = atan c + atan v with v = (u - c) / (1 + u c), |v| <=
// 1/128, and atan v = v - v^3/3 + v^5/5 - v^7/7 (truncation below |v|^9 / 9
// = 1.2e-20); x < 0 adds pi with the sign of y (so y = -0 gives -pi, as
// atan2 does).  A[i] = atan(i/64), i = 0..64, rounded from long double.  The
// reciprocals are the hardware estimate refined by Newton steps: two for
// 1/|t|, one for 1/(1 + u c), whose quotient v is below 1/128.  Within 3 ulp
// of atan2 (4.4e-16 rad) where the host's division stands in for the
// estimate; x = 0 is left to the caller.
constexpr int ATAN_N = 65;

__host__ __device__ inline double rcp_estimate(double b) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_rcp(b);
#else
    return 1.0 / b;
#endif
}

__host__ __device__ inline double atan2_tab(double y, double x, double rx, const double *__restrict__ A) {
    const double t = y * rx;
    const double a = fabs(t);
    const bool flip = a > 1.0;
    const double b = fmax(a, 1.0);
    double r = rcp_estimate(b);
    r = fma(r, fma(-b, r, 1.0), r);
    r = fma(r, fma(-b, r, 1.0), r);
    const double u = flip ? r : a;
    int i = (int)fma(u, 64.0, 0.5);
    i = i < 0 ? 0 : (i > ATAN_N - 1 ? ATAN_N - 1 : i);   // keeps a NaN's index inside the table
    const double c = (double)i * 0.015625;
    const double den = fma(u, c, 1.0);
    double rd = rcp_estimate(den);
    rd = fma(rd, fma(-den, rd, 1.0), rd);
    const double v = (u - c) * rd;
    const double v2 = v * v;
    const double p = v2 * fma(v2, fma(v2, -1.0 / 7.0, 0.2), -1.0 / 3.0);
    const double s = A[i] + fma(v, p, v);
    double res = flip ? (1.5707963267948966 - s) + 6.123233995736766e-17 : s;   // pi/2 as hi + lo
    res = copysign(res, t);
    if (x < 0.0) res = (res + copysign(1.2246467991473532e-16, y)) + copysign(3.141592653589793, y);
    return res;
}

// A tile is a group of up to 64 scan frequencies, one per lane, with
// explicit coordinates (signed row yh, column ix).  The host cuts every
// stored row of G into the runs that fill one 128-byte line (LINE_X = 16
// complex64; a row is N/2 + 1 entries long, so line boundaries move from row
// to row): the head run up to the row's first line boundary, then full
// 16-entry runs, then the tail.  Runs of the same block (head, first full,
// second full, ...) of consecutive rows are packed whole, in row order, into
// tiles of at most 64 lanes spanning at most 8 rows (16 for the SSB pass).
// Each lane's G value then comes from a line no other tile reads, and
// neighbouring lanes see nearly the same lens overlap.
constexpr int LINE_X = 16;
constexpr int MAX_SLOTS = 9;   // fine aliases of one coarse frequency for u <= 3 per axis pair

struct alignas(64) GramTile {
    int nj;              // alias slots: the sorted union of the lanes' offsets (j_y, j_x)
    float rad;           // largest distance of a valid lane's (yh, ix) from (cy, cx), rounded up
    float cy, cx;        // mean (yh, ix) of the valid lanes (cost estimate, centre of the slot test)
    int8_t jy[12], jx[12];
    uint16_t mask[64];   // per lane: bit s set when slot s is an alias of the lane's frequency
    int32_t qidx[64];    // per lane: index of the frequency in the solved list, -1 if none
                         // (preview tiles: 0 for a lane in use; its slots are its fine images)
    int16_t lyh[64];     // per lane: signed row
    int16_t lix[64];     // per lane: column
};

struct alignas(64) SsbTile {
    uint64_t valid;      // lanes inside the band (and inside the stored plane)
    float cy, cx;        // mean (yh, ix) of the valid lanes (cost estimate, centre of the pixel test)
    float rad;           // largest distance of a valid lane's (yh, ix) from (cy, cx), rounded up
    int pad;
    int16_t lyh[64];
    int16_t lix[64];
};

struct OpticsDev {
    double lam, tau_y, tau_x;
    double pt2;      // pi t / (2 lambda), t the depth (0: no depth terms)
    double chi_c[CHI_NCOEF];
};

struct ApertureDev {
    double kc;       // alpha / lambda
    double inv_dk;   // 1 / dk
    double rin2;     // (kc - dk/2)^2 : a == 1 inside (soft)
    double rout2;    // (kc + dk/2)^2 : a == 0 outside (soft); kc^2 (hard)
    double rlim2;    // support is |k|^2 < rlim2: rout2 (soft, strict) or the
                     // next double above kc^2 (hard, |k|^2 <= kc^2)
    // the same in lambda-scaled lengths (|lambda k'|^2 against these)
    double lrlim2;   // lambda^2 rlim2
    double lrin2;    // lambda^2 rin2
    double lkc;      // lambda kc
    double inv_ldk;  // 1 / (lambda dk)
    int soft;
};

// Stream-K decomposition of one Gram launch: the launch's tiles x pixels form
// one linear iteration space (tile-major); wave w takes the contiguous range
// [wbegin[w], wbegin[w+1]) and writes one partial sum per tile segment it
// touches, numbered from seg_off[w].  Tile t's segments are seg_first[t] ..
// seg_first[t+1]-1 (consecutive, in iteration order); the fixup adds them in
// that order, so the result does not depend on scheduling.
struct GramParams {
    const float2 *G;
    const PixelRec *pix;
    const double *tay;         // [n_pix][TAY_N] chi's Taylor coefficients about theta(k)
    const long long *goff;     // [n_pix] element offset of each pixel's plane in G
    int n_pix;
    const GramTile *tiles;
    int N, nh;
    double dq;
    double ldq;                // lambda dq
    ApertureDev ap;
    OpticsDev op;
    double2 *sys;     // [n_q][tri_size(D)] packed augmented systems, slot coordinates
    int a_max, D;
    const long long *wbegin;   // [n_waves + 1]
    const int *seg_off;        // [n_waves]
    const int *seg_first;      // [n_tiles + 1]
    double *partial;           // [n_segments][NACC][64]
    int n_waves;
    const double2 *trig;       // [TRIG_N] (cos, sin)(j pi / 128)
    int slot_test;             // 1: skip slots the per-pixel bound puts out of reach; 0: run all
    int fine_M, fine_mh;       // preview (right sides only): the fine grid M = u N and M / 2 + 1
};

constexpr int MAX_SETS_DEV = 8;   // optics sets of one SSB pass

// SSB pass: stream-K over (band tile, pixel) like the Gram launches, with
// partial sums [n_segments][3 MAXB + 1][64].
struct SsbParams {
    const float2 *G;         // complex64 G, or null with GQ
    const short2 *GQ;        // herm16 G: snorm16 pairs, one scale per pixel
    const float *gscale;     // herm16 scales: [n_bf] by the pixel's plane, or [n_bf][N] by its stored row
    int h16_rows;            // scales per row
    long long plane;         // N (N/2 + 1): plane offset -> pixel index
    const PixelRec *pix;
    const long long *goff;   // [n_pix]
    const double *tay;       // B tables [n_pix][TAY_N] of chi Taylor coefficients about theta(k)
    int n_pix;
    const SsbTile *tiles;
    int N, nh;
    double dq;
    double ldq;              // lambda dq
    int B;
    ApertureDev ap;
    double lam;
    double tau_y[8], tau_x[8];
    double pt2[8];           // pi t_b / (2 lambda) per set
    double chi_c[8][CHI_NCOEF];
    double2 *S_out;          // [B][N][nh] or null
    double *N_out;           // [B][N][nh] or null
    const long long *wbegin; // [n_waves + 1]
    const int *seg_off;      // [n_waves]
    const int *seg_first;    // [n_tiles + 1]
    double *partial;         // [n_segments][3 MAXB + 1][64]
    const double2 *trig;     // [TRIG_N] (cos, sin)(j pi / 128)
};

// Loss path: corrected half planes of a chunk of pixels.
struct CorrParams {
    const float2 *G;
    const PixelRec *pix;       // the chunk's records
    const long long *goff;     // the chunk's plane offsets
    int n_valid;               // pixels in the chunk (planes beyond are zero)
    int N, nh;
    double ldq;                // lambda dq
    ApertureDev ap;
    OpticsDev op;
    const double2 *trig;
    double2 *H;                // [chunk][N][nh] conj(Gamma') G, Gamma' = sqrt(w) Gamma
    double2 *D;                // [chunk] sqrt(w) G(0, k)
};

}  // namespace dsp
