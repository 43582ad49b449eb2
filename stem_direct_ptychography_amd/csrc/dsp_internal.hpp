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

// Horner in theta_x inside Horner in theta_y: 27 FMAs.
__host__ __device__ inline double chi_poly(const double *__restrict__ c, double tx, double ty) {
    double acc = c[chi_off(6)];
#pragma unroll
    for (int j = 5; j >= 0; --j) {
        const double *cj = c + chi_off(j);
        double h = cj[6 - j];
#pragma unroll
        for (int i = 5 - j; i >= 0; --i) h = fma(h, tx, cj[i]);
        acc = fma(acc, ty, h);
    }
    return acc;
}

// ---------------------------------------------------------------------------
// packed upper-triangle index of an n x n matrix, i <= j
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int tri_idx(int i, int j, int n) { return i * (2 * n - i + 1) / 2 + (j - i); }
__host__ __device__ constexpr int tri_size(int n) { return n * (n + 1) / 2; }

// ---------------------------------------------------------------------------
// device tables
// ---------------------------------------------------------------------------
// One active bright-field pixel; 64-byte records so a wave reads one with a
// single scalar load.
struct alignas(64) PixelRec {
    double ky, kx;     // 1/A, scan frame
    double w;          // weight
    double a0;         // aperture a(k)            (pixel-terms kernel)
    double chi0;       // chi(k) of the prepare's optics (pixel-terms kernel)
    long long goff;    // element offset of the pixel's plane in G
    double pad[2];
};

constexpr int TILE_Y = 4;
constexpr int TILE_X = 16;
constexpr int MAX_SLOTS = 9;   // fine aliases of one coarse frequency for u <= 3 per axis pair

// 4 x 16 block of scan frequencies (rows = signed row index, cols = ix); lane
// l holds (yh0 + l / 16, ix0 + l % 16).  The union of the lanes' alias
// offsets (j_y, j_x), sorted, forms the tile's alias slots.
struct alignas(64) GramTile {
    int yh0, ix0;
    int nj;
    int pad0;
    int8_t jy[12], jx[12];
    uint16_t mask[64];   // per lane: bit s set when slot s is an alias of the lane's frequency
    int32_t qidx[64];    // per lane: index of the frequency in the solved list, -1 if none
    int32_t pad1[8];
};

struct alignas(64) SsbTile {
    int yh0, ix0;
    int pad0[2];
    uint64_t valid;      // lanes inside the band (and inside the stored plane)
    int32_t pad1[12];
};

struct OpticsDev {
    double lam, tau_y, tau_x;
    double chi_c[CHI_NCOEF];
};

struct ApertureDev {
    double kc;       // alpha / lambda
    double inv_dk;   // 1 / dk
    double rin2;     // (kc - dk/2)^2 : a == 1 inside (soft)
    double rout2;    // (kc + dk/2)^2 : a == 0 outside (soft); kc^2 (hard)
    int soft;
};

struct GramParams {
    const float2 *G;
    const PixelRec *pix;
    int n_pix;
    const GramTile *tiles;
    int N, nh;
    double dq;
    ApertureDev ap;
    OpticsDev op;
    double2 *sys;     // [n_q][tri_size(D)] packed augmented systems, slot coordinates
    int a_max, D;
};

struct SsbParams {
    const float2 *G;
    const PixelRec *pix;
    const double *chi_tab;   // [B][n_pix]
    int n_pix;
    const SsbTile *tiles;
    int N, nh;
    double dq;
    int B;
    ApertureDev ap;
    double lam;
    double tau_y[8], tau_x[8];
    double chi_c[8][CHI_NCOEF];
    double2 *S_out;          // [B][N][nh] or null
    double *N_out;           // [B][N][nh] or null
    double *partial;         // [n_tiles][B + 1]
};

}  // namespace dsp
