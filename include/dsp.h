/*
 * dsp.h -- regularized direct (single-side-band) ptychography on MI355X.
 *
 * C ABI of libdsp.so.  Plain pointers and sizes only.  Every function returns
 * a dsp_status; nothing throws across the ABI.  On error the outputs are
 * unspecified, no handle is created, an existing handle is unchanged, and
 * dsp_last_error() returns a message (thread-local).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Scan: square N x N (N even, >= 4), step s (A); scan-frequency step
 * dq = 1 / (N s).  Measured data G(q, k) is the Hermitian half plane of the
 * scan-space FFT of each bright-field pixel's intensity trace, complex64,
 * layout [n_bf][N][N/2+1] (pixel-major, contiguous along the last axis),
 * device memory ("Historical WebGPU G(q,k) memory experiment", section
 * "Why herm is exactly lossless").  Stored row iy means signed frequency
 * iy (iy < N/2) or iy - N.
 *
 * Bright-field pixel coordinates k are (k_y, k_x) in 1/A in the scan frame
 * (detector rotation already applied), host double[n_bf][2].  Weights are
 * host double[n_bf] (NULL: all 1).  Only pixels with non-zero aperture
 * weight are used ("active" pixels).
 *
 * Optics: aberration phase in Krivanek polar notation,
 *   chi(k) = (2 pi / lambda) sum C_nm t^(n+1) / (n+1) cos(m (p - phi_nm)),
 *   theta = lambda k + tau, t = |theta|, p = atan2(theta_y, theta_x);
 * probe amplitude A(k) = a(k) exp(-i chi(k)); soft aperture
 * a = clamp(1/2 + (alpha/lambda - |k|) / dk, 0, 1), hard a = [|k| <= alpha/lambda]
 * ("Tilt-corrected SSB on CUDA: fit and preview speed", section "Changes":
 * the soft edge's denominator is the detector step).
 *
 * Weak-object transfer of object frequency Q at pixel k ("Where the 9 s of
 * regularized preparation goes", section "Code path"; "Preparation in one
 * kernel per alias count", section "What changed" 1-2):
 *   L = a(k) a(k-Q) exp(+i [chi(k) - chi(k-Q)]),
 *   R = a(k) a(k+Q) exp(-i [chi(k) - chi(k+Q)]),
 *   T_phi = i (L - R) (phase), T_A = L + R (log-amplitude).
 *
 * Solved frequencies: stored (iy, ix) with ix < N/2, iy != N/2, excluding
 * ix = 0 with signed row <= 0; row-major order; n_q = N (N - 2) / 2 (the
 * 130560 frequencies of a 512 x 512 scan, "Where the 9 s of regularized
 * preparation goes", section "Code path").  Aliases of q on the u-times
 * finer grid (same page, "Code path": the prepare loops over alias counts):
 * K = (iy_signed + j_y N, ix + j_x N) inside [-uN/2, uN/2)^2 with
 * |K|^2 dq^2 < R^2, R = 2 alpha/lambda (+ dk when soft), i.e. the two
 * aperture discs of the transfer's lobes overlap; order (j_y, j_x)
 * ascending; A(q) = number of aliases (1..9).  At the page's 512 x 512,
 * 0.373 A, 30 mrad, upsampling-3 setup this rule gives its alias-count
 * histogram (same page, "Raw numbers": 3770 / 106424 / 19304 / 1062).
 *
 * Asynchrony: validation and host geometry run synchronously in the call;
 * kernels are enqueued on the caller's HIP stream (hipStream_t passed as
 * void*, NULL = the null stream) and results are valid once that stream has
 * passed the call's work.  Device inputs must stay alive and unchanged until
 * then.  Launch or runtime failures return DSP_EDEVICE from the call (or the
 * next call) with HIP's message.  NaN/Inf in G propagate unchecked.
 *
 * Thread safety: one handle per thread; distinct handles are independent.
 * All device memory a handle owns lives on the device current at prepare.
 */
#ifndef DSP_H
#define DSP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSP_OK = 0,
    DSP_EINVAL = 1,        /* bad argument: NULL, size, range, layout */
    DSP_EUNSUPPORTED = 2,  /* valid but not built: odd N, u > 4 */
    DSP_EALIAS = 3,        /* an alias count above the compiled maximum */
    DSP_ENOMEM = 4,        /* device or host allocation failed */
    DSP_EDEVICE = 5        /* HIP runtime / launch failure */
} dsp_status;

typedef enum { DSP_PHASE = 0, DSP_COMPLEX = 1 } dsp_method;

/* One Krivanek term C_{n,m} (A) at angle phi (rad); 1 <= n <= 5,
 * 0 <= m <= n+1, n+1-m even. */
typedef struct {
    int n, m;
    double c_A;
    double phi_rad;
} dsp_aberration;

#define DSP_MAX_ABERRATIONS 16

typedef struct {
    double wavelength_A;     /* lambda */
    double semiangle_rad;    /* alpha */
    double det_step_invA;    /* dk: detector pixel pitch in the scan frame */
    int soft_aperture;       /* 1: soft edge one pixel wide, 0: hard */
    double tilt_rad[2];      /* (tau_y, tau_x) */
    double depth_A;          /* t >= 0: weak object spread evenly through depth t below the
                                plane chi refers to; each lobe gains exp(i h) sinc(h),
                                h = pi t (|theta_k|^2 - |theta_k'|^2) / (2 lambda)
                                ("Where the 9 s of regularized preparation goes", What
                                changed 2); 0: thin object */
    int n_aber;              /* <= DSP_MAX_ABERRATIONS */
    dsp_aberration aber[DSP_MAX_ABERRATIONS];
} dsp_optics;

typedef struct {
    int n_scan;              /* N: square N x N scan, even, >= 4 */
    double step_A;           /* s */
} dsp_scan;

typedef struct {
    dsp_method method;
    int upsampling;          /* u in 1..4 */
    double smoothness_invA;  /* prior p(Q) = (1 + |Q|^2/s^2)^2; <= 0: p = 1 */
    int flags;               /* DSP_FLAG_* */
} dsp_prepare_opts;

#define DSP_FLAG_TIMING 1       /* record HIP events per stage and per Gram launch (read by dsp_info) */
#define DSP_FLAG_COUNT_WORK 2   /* after the prepare's kernels, count the work of each Gram launch
                                   (one extra kernel per launch; read by dsp_info) */
#define DSP_FLAG_NO_SLOT_TEST 4 /* evaluate every alias slot at every pixel: the Gram kernels' per-pixel
                                   slot test (a conservative bound that skips slots out of reach) off.
                                   The systems are bitwise those with the test on; the flag exists to
                                   check that. */

typedef struct dsp_handle dsp_handle;

typedef struct {
    int n_q;                 /* solved frequencies */
    int a_max;               /* largest alias count */
    int n_comp;              /* unknown components: 1 (phase), 2 (complex) */
    int dim;                 /* slot dimension D = n_comp * a_max + 1 */
    int n_bf, n_active_bf;
    int method, upsampling, n_scan;
    int n_tiles;             /* frequency tiles of the Gram kernels: up to 64 frequencies each, cut
                                along G's 128-byte lines (one per lane of a wave) */
    int alias_hist[10];      /* alias_hist[A] = frequencies with A aliases */
    double scale;            /* strength unit: sum of active weights */
    double g_bytes;          /* algorithmic G bytes a prepare reads: n_q * n_active * 8 */
    double lobes;            /* with DSP_FLAG_COUNT_WORK: non-zero weak-object lobes evaluated */
    double host_ms;          /* host time of the prepare call (validation, layout, enqueue) */
    double layout_ms;        /* host time spent building the data-only layout (0 when reused) */
    int layout_cached;       /* 1 when the prepare reused a cached data-only layout */
    double stage_ms[4];      /* with DSP_FLAG_TIMING: pixel terms, Gram, eigenbasis, total */
    int timing_ready;        /* 1 when the timing fields are filled: dsp_info never waits; it
                                fills them once the prepare's work has completed on its stream */
    /* one entry per Gram launch, in launch order (tiles grouped by alias slot
     * count): slot count, tiles and waves; with DSP_FLAG_TIMING the HIP-event
     * duration on the caller's stream; with DSP_FLAG_COUNT_WORK the launch's
     * work summed over its frequencies: [0] aperture-support tests (pixel,
     * alias, lobe), [1] non-zero lobes, [2] non-zero Gram columns (pixel,
     * column), [3] non-zero column pairs c < d, [4] (pixel, frequency) terms.
     * A phase column is non-zero when either lobe is; complex columns are the
     * two lobes. */
    int n_gram_launches;
    int gram_nj[16];
    int gram_tiles[16];
    int gram_waves[16];      /* waves (64-lane workgroups) of the launch */
    double gram_ms[16];
    double gram_fixup_ms[16];/* with DSP_FLAG_TIMING: the launch's partial-sum fixup */
    double gram_work[16][5];
} dsp_info_t;

/*
 * Prepare: per solved frequency, the weighted augmented Gram
 * [T g]^H W [T g] (complex128) -> M = T^H W T, r = T^H W g, P = g^H W g,
 * and, for DSP_PHASE, the eigenbasis of D^-1/2 M D^-1/2 (D = diag(p)), so any
 * strength is a diagonal evaluation ("Where the 9 s of regularized
 * preparation goes", section "Code path").  Complex unknowns are
 * [A_l(Q_1..Q_A), phi(Q_1..Q_A)]; phase unknowns [phi(Q_1..Q_A)].
 *
 * G_c64_dev: device complex64 [n_bf][N][N/2+1], borrowed (not retained).
 * bf_coords_host: double[n_bf][2]; weights_host: double[n_bf] or NULL.
 * Host arrays are copied during the call.  *out receives a new handle that
 * owns its device buffers (free with dsp_destroy).
 */
dsp_status dsp_prepare(const void *G_c64_dev, int n_bf, const double *bf_coords_host,
                       const double *weights_host, const dsp_scan *scan, const dsp_optics *optics,
                       const dsp_prepare_opts *opts, void *hip_stream, dsp_handle **out);

/*
 * Solve at S strengths.  Phase: strengths_host = double[S] (lambda);
 * x = U (c / (Lambda + lambda scale)).  Complex: strengths_host =
 * double[S][2] (lambda_A, lambda_phi); x = (M + scale diag(lambda_A p,
 * lambda_phi p))^-1 r.  ("Where the 9 s ...", section "Code path": complex
 * keeps the Gram and solves at each strength.)
 * x_out_c128_dev: device complex128 [S][n_comp][n_q][a_max]; slot m >= A(q)
 * is written 0.  resid_out_dev: device double[S][n_q] (weighted misfit
 * sum_k w |g - T x|^2) or NULL.
 */
dsp_status dsp_solve(dsp_handle *h, const double *strengths_host, int S, void *x_out_c128_dev,
                     double *resid_out_dev, void *hip_stream);

/*
 * Scatter packed solutions to the fine half plane: spec_out_c128_dev
 * complex128 [S][n_comp][uN][uN/2+1]; alias K lands at (K_y mod uN, K_x)
 * when K_x > 0 or (K_x = 0 and K_y >= 0), otherwise its conjugate lands at
 * -K: the spectrum of a real field at -K is the conjugate of the one at K
 * ("Historical WebGPU G(q,k) memory experiment", section "Why herm is
 * exactly lossless"), and the solved aliases are the object's spectrum on
 * the upsampled grid ("Where the 9 s of regularized preparation goes",
 * sections "Question" and "Code path": upsampling_factor, the per-alias
 * unknowns).  Entries no alias reaches are 0.
 * x_packed_c128_dev: device [S][n_comp][n_q][a_max] from dsp_solve (borrowed).
 * spec_out_c128_dev: device, caller-owned, fully written (zeros included).
 * DSP_EINVAL for a NULL handle or buffer or S <= 0.  Runs on hip_stream.
 */
dsp_status dsp_scatter(const dsp_handle *h, const void *x_packed_c128_dev, int S,
                       void *spec_out_c128_dev, void *hip_stream);

/*
 * SSB / agreement pass over the stored entries (one alias per frequency,
 * Q = q) for B optics sets, reading G once ("Tilt-corrected SSB on CUDA",
 * section "Where the time went": one pass evaluates several parameter sets;
 * "Historical WebGPU G(q,k) memory experiment", section "Object-redraw fast
 * path": the corrected G summed over pixels in Fourier space).
 *   Gamma = T_phi(q, k; set b); S_b(q) = sum_k w conj(Gamma) g;
 *   N_b(q) = sum_k w |Gamma|^2;
 *   E_b = sum_{band, N>0} |S_b|^2 / N_b / sum_{band} sum_k w |g|^2.
 * sets_host: dsp_optics[B], 1 <= B <= 8; the aperture parameters (lambda,
 * alpha, dk, soft) must be equal across sets.  band_invA: double[2] (f_lo,
 * f_hi), inclusive on |q|, or NULL for every stored entry.
 * S_out_c128_dev: complex128 [B][N][N/2+1] or NULL; norm_out_dev: double
 * [B][N][N/2+1] or NULL (entries outside the band are 0);
 * agreement_out_host: double[B] or NULL (non-NULL synchronizes the stream).
 */
dsp_status dsp_ssb(const void *G_c64_dev, int n_bf, const double *bf_coords_host,
                   const double *weights_host, const dsp_scan *scan, const dsp_optics *sets_host,
                   int B, const double *band_invA, void *S_out_c128_dev, double *norm_out_dev,
                   double *agreement_out_host, void *hip_stream);

/*
 * dsp_ssb for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs and errors as dsp_ssb; the results agree with dsp_ssb's
 * to rounding (its stream-K plan may cut the pixel sums into fewer pieces).
 * The call allocates no device memory: no hipMalloc, hipFree or allocating
 * library routine.  Every device buffer of the pass (the layout's pixel,
 * tile and plan tables, copied from host tables the library builds and
 * caches on the host, and the per-call tables and partial sums) is carved
 * from one fixed array of DSP_NOALLOC_SCRATCH_BYTES per device, part of the
 * library's code object: each GPU the library runs on holds it from load
 * until the process ends.  A pass that needs more returns DSP_ENOMEM (with the
 * sizes in dsp_last_error) before any device work; the plan first takes
 * fewer stream-K waves to fit (about 8 sets over 9,000 pixels of a
 * 512 x 512 scan's 0.2-0.9 1/A band fit).  All calls on one GPU share that
 * array, which keeps the last call's contents: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 */
#define DSP_NOALLOC_SCRATCH_BYTES (64ull << 20)
dsp_status dsp_ssb_noalloc(const void *G_c64_dev, int n_bf, const double *bf_coords_host,
                           const double *weights_host, const dsp_scan *scan, const dsp_optics *sets_host,
                           int B, const double *band_invA, void *S_out_c128_dev, double *norm_out_dev,
                           double *agreement_out_host, void *hip_stream);

/*
 * Phase model derived from a prepared complex model, without a pass over G
 * ("Where the 9 s of regularized preparation goes", section "Code path":
 * the complex system contains the phase one).  For every frequency the phase
 * system is the T_phi block of the complex system ([T_A, T_phi] order), the
 * T_phi part of its right side and the same signal power; the phase
 * eigenbasis is then computed as in dsp_prepare.
 *   complex_h: a handle from dsp_prepare with method DSP_COMPLEX (not
 *              modified; it may be destroyed before or after the new handle).
 *   out: a new DSP_PHASE handle, owned by the caller (dsp_destroy), usable with
 *        dsp_solve, dsp_scatter, dsp_info, dsp_export_system, dsp_alias_table.
 * Kernels run on hip_stream; complex_h's prepare must be ordered before them
 * (same stream, or synchronized).  DSP_EINVAL for a NULL argument or a phase
 * source handle; on error *out is NULL.
 */
dsp_status dsp_derive_phase(const dsp_handle *complex_h, void *hip_stream, dsp_handle **out);

/*
 * Two-slot prepared-model cache: one slot per method under the same data and
 * optics key, so phase -> complex -> phase prepares each model once ("Where
 * the 9 s of regularized preparation goes", conclusion 3: a one-slot cache
 * keyed with the method prepares three times; two slots fix it).
 * dsp_cache_get returns the slot's model when its key matches (G's address,
 * g_version, the pixels and weights, scan, optics, upsampling, smoothness
 * and flags, all compared bit for bit), else prepares it (dsp_prepare), or,
 * for DSP_PHASE with derive != 0 while the complex slot holds the same key,
 * derives it from the complex model (dsp_derive_phase), and replaces the
 * slot.
 *   g_version: the caller's generation number of G's contents; change it
 *              when G is rewritten in place.
 *   out: a new reference to the slot's model, owned by the caller: release
 *        it with dsp_destroy.  The model lives until the cache and every
 *        reference handed out have released it, so a reference stays valid
 *        after a later dsp_cache_get replaces its slot or the cache is
 *        destroyed.
 *   how (may be NULL): 1 slot hit, 0 prepared, 2 derived.
 * G is identified by its address and g_version only: a caller that frees G
 * and allocates new data at the same address must pass a new g_version.
 * Calls on one cache are serialized by a lock.  On error the slot keeps its
 * model and *out is NULL; errors as dsp_prepare and dsp_derive_phase.
 */
typedef struct dsp_cache dsp_cache;
dsp_status dsp_cache_create(dsp_cache **out);
void dsp_cache_destroy(dsp_cache *c);
dsp_status dsp_cache_get(dsp_cache *c, const void *G_c64_dev, unsigned long long g_version, int n_bf,
                         const double *bf_coords_host, const double *weights_host, const dsp_scan *scan,
                         const dsp_optics *optics, const dsp_prepare_opts *opts, int derive, void *hip_stream,
                         dsp_handle **out, int *how);

/*
 * Compact G ("Historical WebGPU G(q,k) memory experiment", compact preview /
 * herm16): the stored half plane of each pixel as pairs of signed
 * normalized 16-bit integers and one float scale per pixel, or with
 * row_scales one per stored row (same page, "Conclusions": per-q-row block
 * scales, n per pixel, resolve the weak high-q tail).  With s the pixel's
 * (or the row's) scale:
 *   s = max over the pixel's plane (row) of |G| (|G|^2 = re^2 + im^2 in
 *       FP64, the root rounded to float);
 *   Q[k][iy][ix][c] = floor(0.5 + 32767 clamp(v / s, -1, 1)) for the
 *       components v = Re G, Im G (FP64; 0 where s = 0);
 *   G is read back as max(Q / 32767, -1) * s.
 * G_c64_dev: complex64 [n_bf][n_scan][n_scan/2+1]; Q_i16_dev: int16
 * [n_bf][n_scan][n_scan/2+1][2]; scale_dev: float [n_bf], or [n_bf][n_scan]
 * with row_scales; all device, caller-owned, G 16-byte and Q 8-byte aligned
 * (as any device allocation is).  Runs on hip_stream.
 * DSP_EINVAL for NULL or misaligned pointers, n_bf <= 0, odd or too small
 * n_scan.
 */
dsp_status dsp_quantize_herm16(const void *G_c64_dev, int n_bf, int n_scan, int row_scales, void *Q_i16_dev,
                               float *scale_dev, void *hip_stream);

/* dsp_ssb over herm16 G (Q and scale from dsp_quantize_herm16, half the
 * bytes of complex64 G; row_scales as given to it): same arguments, outputs
 * and errors as dsp_ssb. */
dsp_status dsp_ssb_herm16(const void *Q_i16_dev, const float *scale_dev, int row_scales, int n_bf,
                          const double *bf_coords_host, const double *weights_host, const dsp_scan *scan,
                          const dsp_optics *sets_host, int B, const double *band_invA, void *S_out_c128_dev,
                          double *norm_out_dev, double *agreement_out_host, void *hip_stream);

/* Sizes, histogram, timings of a prepared handle.  Does not wait for the
 * device, except to read DSP_FLAG_COUNT_WORK counts (a blocking copy). */
dsp_status dsp_info(const dsp_handle *h, dsp_info_t *out);

/*
 * Parity export.  aug_out_c128_dev: complex128 [n_q][D][D], the Hermitian
 * augmented system in slot coordinates: unknown (component c, alias m) at
 * index c * a_max + m, g at index D - 1; rows/columns of absent aliases are 0.
 * eig_out_dev: double [n_q][a_max] ascending eigenvalues (phase), or NULL.
 */
dsp_status dsp_export_system(const dsp_handle *h, void *aug_out_c128_dev, double *eig_out_dev,
                             void *hip_stream);

/* Host copies of the handle's alias table (the frequencies and their
 * aliases defined above: "Where the 9 s of regularized preparation goes",
 * sections "Code path" and "Raw numbers"): q_host int32[n_q][2] (iy, ix),
 * count_host int32[n_q], K_host int32[n_q][a_max][2] (0 past A(q)).  Any
 * pointer may be NULL (not written); all are caller-owned host memory.  No
 * device call.  DSP_EINVAL for a NULL handle. */
dsp_status dsp_alias_table(const dsp_handle *h, int32_t *q_host, int32_t *count_host, int32_t *K_host);

/* Releases a reference to a handle (NULL is ignored); the handle is freed
 * with its last reference (dsp_prepare and dsp_derive_phase create one, and
 * a cache holds one per slot and hands out one per dsp_cache_get).  Its
 * device buffers (one block per handle) go back to the library's per-device
 * cache behind events recorded after the last work queued with them on each
 * stream the handle was used on; the call does not wait for the device, and
 * a later prepare reuses the block after making its own stream wait on those
 * events.  The cache keeps at most 4 GiB per device (older blocks are then
 * freed) and gives its blocks back when an allocation would otherwise fail. */
void dsp_destroy(dsp_handle *h);
const char *dsp_last_error(void);

/* ---------------- host-only geometry (no device calls) ---------------- */

/* n_q, a_max and alias histogram hist_out[10] (may be NULL) of a scan. */
dsp_status dsp_geometry_counts(const dsp_scan *scan, const dsp_optics *optics, int upsampling,
                               int *n_q, int *a_max, int32_t *hist_out);

/* Solved frequencies and their aliases (the rule above; "Where the 9 s of
 * regularized preparation goes", sections "Code path" and "Raw numbers"),
 * same layout as dsp_alias_table (K_host sized n_q * a_max * 2 with a_max
 * from dsp_geometry_counts).  Host only; errors as dsp_geometry_counts. */
dsp_status dsp_alias_geometry(const dsp_scan *scan, const dsp_optics *optics, int upsampling,
                              int32_t *q_host, int32_t *count_host, int32_t *K_host);

/* Active bright-field pixels: those with non-zero aperture weight a(k) > 0
 * ("Historical WebGPU G(q,k) memory experiment", section "Gotchas recorded": the
 * active set, not the labelled set, carries signal), in input order.
 * bf_coords_host double[n_bf][2]; idx_out int32[n_bf] (caller-owned; may be
 * NULL to count only); *n_active receives the count.  Host only.
 * DSP_EINVAL for bad optics, n_bf < 0, NULL coordinates or NULL n_active. */
dsp_status dsp_active_bf(const double *bf_coords_host, int n_bf, const dsp_optics *optics,
                         int32_t *idx_out, int *n_active);

/* Stored entries with f_lo <= |q| <= f_hi (the SSB band). */
dsp_status dsp_band_count(const dsp_scan *scan, const double *band_invA, int *count);

/* The library's chi(k) (its polynomial expansion of the Krivanek terms)
 * evaluated on the host at n points k_host double[n][2]: chi_out double[n]. */
dsp_status dsp_chi_host(const dsp_optics *optics, const double *k_host, int n, double *chi_out);

/* Upsampled SSB preview: the object fast path ("Historical WebGPU G(q,k)
 * memory experiment", section "Object-redraw fast path": the corrected G
 * summed over the bright-field pixels in Fourier space, then one inverse FFT
 * and one angle; "Tilt-corrected SSB on CUDA: fit and preview speed",
 * section "Changes": the 1x and 3x drag previews).  On the fine grid
 * M = u N, for every K != 0 of its half plane (signed row, column 0..M/2):
 *   P(K) = i sum_k w_k conj(Gamma(K, k)) G(K mod N, k),  Gamma = T_phi at Q = K dq,
 * over the active pixels (G(-q) = conj G(q) supplies q beyond column N/2),
 * and P(0) = sum_k w_k G(0, k); P = 0 on the fine Nyquist row and column
 * (index M/2 stands for +-M/2 dq, whose corrections differ).  The corrected spectrum of a real image is
 * anti-Hermitian off DC (same page, section "Open"): the full plane has
 * P(-K) = -conj P(K), the object is o = ifft2(full plane), the phase angle(o).
 *   G_c64_dev, n_bf, bf_coords_host, weights_host, scan, optics: as dsp_ssb
 *       with one optics set (depth terms included).
 *   upsampling: u in 1..4.
 *   spec_out_c128_dev: [M][M/2+1] complex128 P, or NULL.
 *   phase_out_dev: [M][M] float64 phase (rad, in [-pi, pi]), or NULL; at
 *       least one output.
 * Asynchronous on hip_stream; scratch from the stream's arena.  The inverse
 * FFT is hipFFT's Z2D; its plan per (device, M) is kept until the process
 * ends.  DSP_EUNSUPPORTED for u outside 1..4, DSP_EINVAL for bad arguments,
 * DSP_EDEVICE for a hipFFT failure. */
dsp_status dsp_preview(const void *G_c64_dev, int n_bf, const double *bf_coords_host, const double *weights_host,
                       const dsp_scan *scan, const dsp_optics *optics, int upsampling, void *spec_out_c128_dev,
                       double *phase_out_dev, void *hip_stream);

/* Loss path: every active pixel's own object and their phase moments
 * ("Tilt-corrected SSB on CUDA: fit and preview speed", section "Changes",
 * loss path: each pixel's corrected full plane straight from its stored half
 * plane, an unscaled inverse FFT, and phase moments reduced as the angles are
 * read; "Historical WebGPU G(q,k) memory experiment", section "Object-redraw
 * fast path": mean(angle(object)) needs the per-pixel phases).  Pixel k's
 * corrected plane is C_k(q) = i w_k conj(Gamma(q, k)) G(q, k) for q != 0
 * (zero on the Nyquist row and column) and w_k G(0, k) at DC; its object
 * o_k = ifft2(C_k) and theta_k = angle(o_k).  Outputs:
 *   mean_phase_out_dev: [N][N] float64 sum_k w_k theta_k / sum_k w_k, or NULL;
 *   loss_out_host: the mean over the scan of sum_k w_k (theta_k - mean)^2 /
 *       sum_k w_k, or NULL (non-NULL synchronizes the stream).
 * Arguments as dsp_preview (u = 1).  G's self-conjugate column (ix = 0)
 * should hold conjugate pairs G(-q) = conj G(q), as a real transform gives.
 * For power-of-two N from 8 to 1024 two fused passes take the planes through
 * the inverse real transform (self-sorting radix-8 transforms in LDS: a
 * column pass that computes the corrected values, a row pass that goes on
 * to the phases and their moments), and neither the corrected planes' second
 * read nor the real images reach memory; they read the self-conjugate
 * columns as given.  Other N write the corrected planes for chunks of pixels
 * (about 1 GB per batch, from the stream's arena), run hipFFT's batched Z2D
 * (plans kept until the process ends; it uses those columns' Hermitian
 * part) and reduce the moments.  DSP_EINVAL for bad arguments or weights
 * summing to zero, DSP_EDEVICE for a hipFFT failure. */
dsp_status dsp_loss(const void *G_c64_dev, int n_bf, const double *bf_coords_host, const double *weights_host,
                    const dsp_scan *scan, const dsp_optics *optics, double *mean_phase_out_dev, double *loss_out_host,
                    void *hip_stream);

/* The phase differences of the transfer's two lobes as the Gram kernels form
 * them (the same source: chi expanded about theta(k) = lambda k + tau, one
 * evaluation of its even and odd parts in d = lambda Q for both lobes),
 * evaluated on the host.  k_host and q_host double[2 n] (ky, kx) and
 * (Qy, Qx) in 1/A, scan frame; out double[2 n]: (chi(k - Q) - chi(k),
 * chi(k + Q) - chi(k)): the phases of the lobes L and R of the weak-object
 * transfer above ("Where the 9 s of regularized preparation goes", section
 * "Code path").  EINVAL on bad optics or NULL buffers. */
dsp_status dsp_chi_shift_host(const dsp_optics *optics, const double *k_host, const double *q_host, int n,
                              double *out);

/* The library's FP64 sine and cosine of the transfer's phase factors (the
 * same source the kernels compile) evaluated on the host at n points:
 * x_host double[n] -> sin_out, cos_out double[n]. */
dsp_status dsp_sincos_host(const double *x_host, int n, double *sin_out, double *cos_out);

/* The loss path's FP64 atan2 (table-reduced, for phases whose x is fixed per
 * pixel; the same source the kernels compile, with the host's division in
 * place of the hardware reciprocal estimate) at n points: y_host, x_host
 * double[n] -> out double[n]; x = 0 takes the C library's atan2, as the
 * kernels do.  DSP_EINVAL for n < 0 or NULL arrays with n > 0. */
dsp_status dsp_atan2_host(const double *y_host, const double *x_host, int n, double *out);

#ifdef __cplusplus
}
#endif

#endif /* DSP_H */
