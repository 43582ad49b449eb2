// Kernel parameter blocks and launchers of libdsp (internal).
#pragma once

#include "dsp_internal.hpp"

namespace dsp {

struct EigParams {
    const double2 *sys;   // packed systems [n_q][tri_size(D)]
    int D, a_max;
    const int32_t *qlist; // frequencies with this alias count
    int n;
    const double *prior;  // [n_q][a_max]
    double *lam;          // [n_q][a_max]
    double2 *U;           // [n_q][a_max][a_max]
    double2 *c;           // [n_q][a_max]
};

struct SolveParams {
    const double2 *sys;
    int D, a_max, n_q;
    const int32_t *qlist;
    int n;
    const double *prior;
    const double *lam;
    const double2 *U;
    const double2 *c;
    double strengths[64];     // by value: phase [S] (S <= 64), complex [S][2] (S <= 32)
    int S;
    double scale;
    double2 *x;               // [S][n_comp][n_q][a_max]
    double *resid;            // [S][n_q] or null
};

struct ScatterParams {
    const double2 *x;         // [SC][n_q][a_max]
    int SC, n_q, a_max;
    const int32_t *count;     // [n_q]
    const int32_t *K;         // [n_q][a_max][2]
    int nf;                   // u N
    double2 *spec;            // [SC][nf][nf/2+1]
};

hipError_t launch_pixel_terms(const PixelBase *in, PixelRec *out, int n_pix, const ApertureDev &ap, const OpticsDev &op,
                              double *chi_tab, int chi_stride, double *tay, hipStream_t st);
// Gram launches: method DSP_PHASE (0), DSP_COMPLEX (1), or GRAM_PREVIEW (2):
// right sides only, one per alias slot, written into the preview's fine half
// plane (GramParams::sys then points at it; fine_M, fine_mh give its shape).
constexpr int GRAM_PREVIEW = 2;
constexpr int MAX_NJ_PREVIEW = 9;
int gram_nacc(int nj, int method);   // doubles per lane of one partial sum
hipError_t gram_occupancy(int nj, int method, int *blocks_per_cu);
hipError_t launch_gram(const GramParams &prm, int nj, int method, int n_waves, hipStream_t st);
hipError_t launch_gram_fixup(const GramParams &prm, int nj, int method, int n_tiles, hipStream_t st);
hipError_t launch_work_count(const GramParams &prm, int method, int n_tiles, unsigned long long *out,
                             hipStream_t st);
hipError_t launch_herm16(const float2 *G, int n_bf, int N, int nh, bool rows, short2 *Q, float *scale,
                         hipStream_t st);
hipError_t launch_phase_from_complex(const double2 *csys, double2 *psys, int a_max, int n_q, hipStream_t st);
hipError_t launch_eig(const EigParams &prm, int A, hipStream_t st);
hipError_t launch_solve(const SolveParams &prm, int A, int method, hipStream_t st);
hipError_t launch_fill_zero(double *p, size_t n, hipStream_t st);
hipError_t launch_scatter(const ScatterParams &prm, hipStream_t st);
hipError_t launch_export(const double2 *sys, int n_q, int D, double2 *dense, hipStream_t st);
int ssb_maxb(int B);                 // compiled set count used for B sets
int ssb_nacc(int maxb);              // doubles per lane of one SSB partial sum
hipError_t ssb_occupancy(int maxb, int *blocks_per_cu);
// SSB kernel over n_waves stream-K ranges, then per-tile reduction and
// write-out; tile_part receives [n_tiles][MAXB + 1] agreement partials.
hipError_t launch_preview_dc(const PixelBase *pix, const long long *goff, int n_pix, const float2 *G, double2 *dc,
                             hipStream_t st);
hipError_t launch_preview_spectrum(const double2 *S, const double2 *dc, long long n, double2 *P, hipStream_t st);
hipError_t launch_preview_phase(double *img, long long n, const double2 *dc, hipStream_t st);
hipError_t launch_corrected_half(const CorrParams &prm, int n_planes, hipStream_t st);
hipError_t launch_phase_moments(const double *img, const double2 *D, const PixelBase *pb, int cn, long long nn,
                                double *s1, double *s2, hipStream_t st);
int loss_blocks(long long nn);
// Fused loss pass over one chunk of cn pixels (power-of-two N, 8 <= N <= 1024):
// column transform with the corrected values (Y into prm.H, D into prm.D),
// row transform with the phase moments into ng group partials, then
// s1/s2 += the partials.  tw: e^{+2 pi i m / N}, m < N/2; atab: atan(i/64),
// i = 0..ATAN_N - 1 (atan2_tab).
int loss_fused_cols(int N);
hipError_t launch_loss_fused(const CorrParams &prm, const double2 *tw, const double *atab, int cn, const PixelBase *pb,
                             int ng, double *s1p, double *s2p, double *s1, double *s2, hipStream_t st);
hipError_t launch_loss(const double *s1, const double *s2, long long nn, double W, double *mean_out, double *part,
                       double *loss, hipStream_t st);
hipError_t launch_ssb(const SsbParams &prm, int n_waves, int n_tiles, double *tile_part, hipStream_t st);
int ssb_partial_stride(int B);
hipError_t launch_agreement(const double *partial, int n_tiles, int B, double *E, hipStream_t st);

// Fixed per-device scratch of the allocation-free SSB pass (dsp_ssb_noalloc):
// *out receives the current device's copy (hipGetSymbolAddress, once per
// device; no allocation).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
hipError_t noalloc_scratch(char **out);

constexpr int MAX_NJ_PHASE = 8;
constexpr int MAX_NJ_COMPLEX = 6;
constexpr int MAX_A_SOLVE_COMPLEX = 6;
constexpr int MAX_A_PHASE = 8;
constexpr int MAX_SETS = 8;

}  // namespace dsp
