/*
 * hyena.h -- C ABI of the MI355X (gfx950) Hyena operator library, libhyena.so.
 *
 * The Hyena operator is the data-parallel core of a StripedHyena 2 (Evo 2)
 * mixer.  Per channel c it computes
 *
 *     u      = x1 * v                                   (input gate)
 *     h[t]   = sum_n R[c,n] * exp(lam[c,n] * t)          (modal long filter)
 *     z[t]   = sum_{k<=t} h[t-k] * u[k]                  (causal convolution)
 *     y      = x2 * z + skip[c] * u                      (output gate + skip)
 *
 * Sources on the pages:
 *  - three streams from the 3H input projection and a gated output that feeds
 *    out_proj: evo2_flash README, layer_names table ('blocks.N.projections',
 *    'blocks.N.filter');
 *  - hcl blocks are a modal-form IIR filter evaluated with an FFT, hcm / hcs
 *    blocks are FIR filters of inner length 128 / 7: Evo2-7B-262K model card,
 *    Implementation Notes, 'Block dispatch';
 *  - log_poles / residues are kept in fp32, everything else is bf16:
 *    Evo2-7B-262K model card, Usage, 'Note on dtype' and Implementation Notes;
 *  - bf16 is mandatory because the residual stream reaches ~1e12: evo2_flash
 *    README, Requirements and install;
 *  - the per-layer inference cache holds the FIR window and the IIR modal
 *    state: Evo2-7B-262K model card, Implementation Notes, 'Custom cache';
 *    Evo1-1.5-7B-8K model card, Implementation Notes, 'Cache subclass';
 *  - chunked prefill must give the single-pass result, whatever the chunk
 *    size: TurboQuant-Bio int4 Evo 2 checkpoints, 'Important: a correctness
 *    fix comes with this' and 'Chunk size'.
 *
 * Conventions shared by every entry point
 *  - Activations x1, x2, v, y are channel-major (B, D, L) contiguous arrays
 *    (time is the fastest axis) of element type `io`: HYENA_F32 (float) or
 *    HYENA_BF16 (bfloat16 bit patterns, 2 bytes).  Arithmetic is fp32; y is
 *    rounded once, to nearest even.
 *  - Parameters are fp32 and shared across the batch: log_poles and residues
 *    (D, N), skip (D) (NULL means 0), taps (D, K) with taps[c*K + k] the
 *    coefficient of lag k (PyTorch conv1d weights are the reverse order).
 *  - The modal state is fp32 (B, D, N): state[b, c, n] = s_n(t) =
 *    sum_{k<=t} p_n^(t-k) u[k], p_n = exp(lam[c,n]), after the last token.
 *  - Every pointer argument is a DEVICE pointer of the current HIP device.
 *    The caller allocates and frees all memory.  Inputs are read only; outputs
 *    must not overlap inputs (except state_out == state_in, which is allowed).
 *    Base pointers must be aligned to their element size; 16-byte alignment
 *    enables the vectorised paths.
 *  - `stream` is the HIP stream the call is enqueued on (NULL = the null
 *    stream).  Every call is asynchronous on that stream and never synchronises the
 *    host; device faults surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before any launch.  Nothing is
 *    printed and nothing throws across the ABI.  Sizes of 0 are accepted and
 *    do nothing (except hyena_chunk_fwd with L = 0, which copies state_in to
 *    state_out, or zeroes it when state_in is NULL).  Non-finite inputs
 *    propagate to the outputs; they are not an error.
 *  - The library allocates nothing; apart from the device scratch of
 *    hyena_fftconv_fwd_noalloc (below) it keeps no global or per-device
 *    state.  All entry points are reentrant and may be called from several
 *    host threads.  No entry point allocates, clears memory with a memset or
 *    synchronises, so every one may be captured into a HIP graph and
 *    replayed (the pointers it was captured with stay in use).
 */
#ifndef HYENA_H_
#define HYENA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYENA_ABI_VERSION 8

typedef enum hyena_status {
    HYENA_OK = 0,
    HYENA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad enum, misalignment, N out of [1, 64] */
    HYENA_ERR_UNSUPPORTED = 2,   /* valid but beyond what this build implements (limits below) */
    HYENA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the entry point's *_workspace_size() */
    HYENA_ERR_LAUNCH = 4,        /* a HIP launch or runtime call failed (hipGetLastError) */
} hyena_status_t;

typedef enum hyena_dtype {
    HYENA_F32 = 0,
    HYENA_BF16 = 1,
} hyena_dtype_t;

/* Algorithm of hyena_chunk_fwd_algo, hyena_chunk_fwd_cpx_algo and
 * hyena_chunk_fwd_tokmajor_algo (the entry points without the suffix take
 * AUTO).  Every algorithm computes the same function. */
typedef enum hyena_chunk_algo {
    HYENA_CHUNK_AUTO = 0,        /* MFMA when the modes fit it (below), else FFT;
                                    token-major: see hyena_chunk_fwd_tokmajor */
    HYENA_CHUNK_FFT = 1,         /* per chunk: zero-padded FFT of length 2C + modal state terms
                                    (channel-major entries only) */
    HYENA_CHUNK_MFMA = 2,        /* blocked Toeplitz on bf16x3 MFMA + modal state scan;
                                    N <= 32 real or N <= 16 complex modes */
    HYENA_CHUNK_RECURRENCE = 3,  /* per token, the modal state recurrence over segments
                                    run in parallel (token-major entry only) */
} hyena_chunk_algo_t;

/* Limits of this build. */
#define HYENA_MAX_MODES 64               /* N */
#define HYENA_MAX_FIR_TAPS 1024          /* K */
#define HYENA_MAX_FIR_TAPS_TOKMAJOR 128  /* K of hyena_fir_fwd_tokmajor */
#define HYENA_MAX_FFT_LEN (1 << 20)      /* single-pass FFT length, next pow2 >= 2L */
#define HYENA_MAX_FFT_CHUNK 8192         /* C for HYENA_CHUNK_FFT (FFT length 2C <= 16384) */
#define HYENA_NOALLOC_SCRATCH_BYTES (64u << 20)  /* device scratch of hyena_fftconv_fwd_noalloc */

int hyena_abi_version(void);
const char* hyena_status_string(hyena_status_t status);

/*
 * hyena_modal_filter -- materialise the modal long filter.
 *   h[c, t] = sum_{n<N} residues[c, n] * exp(log_poles[c, n] * t),  0 <= t < L,
 * evaluated in fp32 with exp taken directly (no long power recurrence).
 * The modal form and its fp32 parameters: Evo2-7B-262K model card,
 * Architecture ('Training dtype') and Implementation Notes ('log_poles /
 * residues kept in fp32'); Evo1-1.5-7B-8K model card, Architecture.
 *   log_poles, residues : (D, N) fp32, device
 *   h                   : (D, L) fp32, device, written
 * The fused entry points below generate h on chip and never call this; it
 * exists as a building block and for tests.
 */
hyena_status_t hyena_modal_filter(const float* log_poles, const float* residues,
                                  int64_t D, int64_t N, int64_t L,
                                  float* h, hipStream_t stream);

/*
 * hyena_fir_fwd -- gated explicit-FIR Hyena operator (hcs: K = 7, hcm: K = 128).
 *   z[t] = sum_{k<K, k<=t} taps[c, k] * u[t-k],   u = x1 * v,
 *   y    = x2 * z + skip[c] * u.
 * Evo2-7B-262K model card, Implementation Notes, 'Block dispatch' (FIR
 * cascades of inner length 128 and 7); only the single FIR is implemented.
 *   x1, x2, v : (B, D, L) `io`, device;  y : (B, D, L) `io`, device, written
 *   taps      : (D, K) fp32, device, 1 <= K <= HYENA_MAX_FIR_TAPS
 *   skip      : (D) fp32, device, or NULL
 */
hyena_status_t hyena_fir_fwd(const void* x1, const void* x2, const void* v,
                             const float* taps, int64_t K, const float* skip,
                             void* y, int64_t B, int64_t D, int64_t L,
                             hyena_dtype_t io, hipStream_t stream);

/*
 * hyena_fftconv_fwd -- single-pass modal Hyena operator.
 * The causal convolution is a zero-padded FFT product of length
 * Nfft = next power of two >= 2L ('modal-form IIR via FFT': Evo2-7B-262K
 * model card, Implementation Notes, 'Block dispatch'; 'FFT-based long
 * convolution': Evo1-1.5-7B-8K model card, Implementation Notes, 'Hyena
 * engine').  h is generated on chip; it never touches memory.
 *   x1, x2, v : (B, D, L) `io`;  y : (B, D, L) `io`, written
 *   log_poles, residues : (D, N) fp32, 1 <= N <= HYENA_MAX_MODES
 *   skip : (D) fp32 or NULL
 *   workspace : device buffer of at least hyena_fftconv_workspace_size(...)
 *               bytes, 16-byte aligned, owned by the caller, contents
 *               scratch (may be NULL when that size is 0).  Rows with
 *               L <= 4096 are transformed on chip and need none; rows with
 *               4096 < L <= 32768 hand one half-transform between two
 *               launches through it (2 * Nfft bytes per row); longer rows go
 *               through the four-step path (8 * Nfft bytes per row).  Either
 *               way rows are processed in batches of at most 1 GiB of
 *               workspace.  Calls sharing one workspace must be ordered
 *               (same stream).
 * Nfft > HYENA_MAX_FFT_LEN -> HYENA_ERR_UNSUPPORTED; workspace NULL, short or
 * misaligned when one is needed -> HYENA_ERR_WORKSPACE.
 */
hyena_status_t hyena_fftconv_fwd(const void* x1, const void* x2, const void* v,
                                 const float* log_poles, const float* residues,
                                 int64_t N, const float* skip, void* y,
                                 int64_t B, int64_t D, int64_t L, hyena_dtype_t io,
                                 void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * hyena_fftconv_fwd_noalloc -- hyena_fftconv_fwd for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  It takes no workspace; rows that need one
 * (L > 4096) go through a scratch array of HYENA_NOALLOC_SCRATCH_BYTES (64
 * MiB) that is part of the library's device code: every GPU the library is
 * loaded on holds its own copy from the load until the process ends.  Its
 * address on a device is looked up on the first call there and kept.  Rows
 * are processed in batches that fit the scratch (fewer rows per launch than
 * hyena_fftconv_fwd at L > 4096, the same results bit for bit); a shape
 * whose single row needs more than the scratch -> HYENA_ERR_UNSUPPORTED
 * (none within HYENA_MAX_FFT_LEN: the longest row needs 8 MiB).  The
 * scratch's contents are left from the last call and nothing in it needs to
 * start at zero.  All calls on one GPU share the scratch: calls that overlap
 * in time on one GPU (different streams without ordering between them) race
 * and give wrong results; calls on one stream are ordered.  Arguments,
 * layouts and errors are otherwise those of hyena_fftconv_fwd; no memory is
 * allocated and nothing synchronises.
 */
hyena_status_t hyena_fftconv_fwd_noalloc(const void* x1, const void* x2, const void* v,
                                         const float* log_poles, const float* residues,
                                         int64_t N, const float* skip, void* y,
                                         int64_t B, int64_t D, int64_t L, hyena_dtype_t io,
                                         hipStream_t stream);

/* Workspace bytes hyena_fftconv_fwd needs for this shape: 0 when one launch
 * transforms the rows on chip (L <= 4096) or the shape is empty or
 * unsupported. */
size_t hyena_fftconv_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N,
                                    hyena_dtype_t io);

/*
 * hyena_chunk_fwd -- chunked prefill with the modal state carried in and out.
 * The sequence is processed in chunks [t0, t0 + C') of C tokens (the last
 * may be shorter); within a chunk
 *   z[t] = sum_{k=t0}^{t} h[t-k] u[k] + sum_n R_n p_n^(t-t0+1) s_n,
 * and after it  s_n <- p_n^C' s_n + sum_j p_n^(C'-1-j) u[t0+j].
 * The output equals the single-pass output of the whole sequence started from
 * the state `state_in` (TurboQuant-Bio int4 Evo 2 checkpoints, 'Important: a
 * correctness fix comes with this' and 'Chunk size'); the IIR modal state is
 * the layer's inference cache (Evo2-7B-262K model card, Implementation Notes,
 * 'Custom cache'; Evo1-1.5-7B-8K model card, Implementation Notes, 'Cache
 * subclass').  All chunks of the call run in ONE launch; L = C gives one
 * chunk per call and L = C = 1 is a decode step.
 *   x1, x2, v : (B, D, L) `io`;  y : (B, D, L) `io`, written
 *   log_poles, residues : (D, N) fp32;  skip : (D) fp32 or NULL
 *   state_in  : (B, D, N) fp32 or NULL (zero state)
 *   state_out : (B, D, N) fp32, written (may equal state_in)
 *   C >= 1.  The algorithm is HYENA_CHUNK_AUTO: the matrix-core blocked
 *   Toeplitz for N <= 32 modes, else per-chunk FFTs (then C' <=
 *   HYENA_MAX_FFT_CHUNK, else HYENA_ERR_UNSUPPORTED).
 */
hyena_status_t hyena_chunk_fwd(const void* x1, const void* x2, const void* v,
                               const float* log_poles, const float* residues,
                               int64_t N, const float* skip,
                               const float* state_in, float* state_out,
                               void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                               hyena_dtype_t io, hipStream_t stream);

/*
 * hyena_chunk_fwd_algo -- hyena_chunk_fwd with the algorithm chosen by the
 * caller (same function, same arguments, same errors):
 *   HYENA_CHUNK_AUTO  as hyena_chunk_fwd;
 *   HYENA_CHUNK_FFT   per chunk a zero-padded FFT product of length 2C', any
 *                     N, C' <= HYENA_MAX_FFT_CHUNK;
 *   HYENA_CHUNK_MFMA  blocked Toeplitz on the matrix cores, any C, N <= 32
 *                     (N > 32 -> HYENA_ERR_UNSUPPORTED);
 *   anything else -> HYENA_ERR_INVALID_ARG.
 */
hyena_status_t hyena_chunk_fwd_algo(const void* x1, const void* x2, const void* v,
                                    const float* log_poles, const float* residues,
                                    int64_t N, const float* skip,
                                    const float* state_in, float* state_out,
                                    void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                                    hyena_dtype_t io, hyena_chunk_algo_t algo,
                                    hipStream_t stream);

/*
 * hyena_modal_decode -- one decode step of the modal operator from its cache.
 * The hcl block's inference cache is its modal state (Evo2-7B-262K model
 * card, Implementation Notes, 'Custom cache'; Evo1-1.5-7B-8K model card,
 * Implementation Notes, 'Cache subclass').  For one token per (b, c):
 *   s_n <- p_n s_n + u,  u = x1 v,  p_n = exp(log_poles[c, n]),
 *   y = x2 * sum_n R_n s_n + skip * u,  rounded once to `io`.
 * Equal to hyena_chunk_fwd with L = 1, without its per-row set-up.
 *   x1, x2, v : (B, D) `io` (one token);  y : (B, D) `io`, written
 *   log_poles, residues : (D, N) fp32, 1 <= N <= HYENA_MAX_MODES
 *   skip : (D) fp32 or NULL
 *   state_in  : (B, D, N) fp32 or NULL (empty prefix)
 *   state_out : (B, D, N) fp32, written (may equal state_in)
 */
hyena_status_t hyena_modal_decode(const void* x1, const void* x2, const void* v,
                                  const float* log_poles, const float* residues,
                                  int64_t N, const float* skip,
                                  const float* state_in, float* state_out,
                                  void* y, int64_t B, int64_t D, hyena_dtype_t io,
                                  hipStream_t stream);

/*
 * hyena_fir_fwd_window -- explicit FIR continuing a sequence from its cache.
 * The hcm / hcs blocks' inference cache is the window of their last K-1
 * inputs u (Evo2-7B-262K model card, Implementation Notes, 'Custom cache';
 * Evo1-1.5-7B-8K model card, Implementation Notes, 'Cache subclass').  With
 * e = [window_in, u[0:L)]:
 *   z[t] = sum_{k<K} w[c, k] e[K-1+t-k],  y = x2 * z + skip * u,
 * and window_out = the last K-1 entries of e.  Any L >= 0 (L = 1 per decode
 * step, L < K-1 included); successive calls with the window handed over
 * equal one call over the whole sequence.
 *   x1, x2, v, taps, K, skip, y, B, D, L, io : as hyena_fir_fwd
 *   window_in  : (B, D, K-1) fp32, oldest first, or NULL (fresh sequence)
 *   window_out : (B, D, K-1) fp32, written (may equal window_in); may be
 *                NULL only when K = 1
 * L = 0 moves window_in to window_out (zeros when window_in is NULL).
 */
hyena_status_t hyena_fir_fwd_window(const void* x1, const void* x2, const void* v,
                                    const float* taps, int64_t K, const float* skip,
                                    const float* window_in, float* window_out,
                                    void* y, int64_t B, int64_t D, int64_t L,
                                    hyena_dtype_t io, hipStream_t stream);

/*
 * Complex-pole modal filters.  Evo 1's Hyena filter is given by modal-form
 * poles / residues with a Hyena state size of 8, kept in fp32 (Evo1-1.5-7B-8K
 * model card, Architecture).  The entry points below take the poles in log
 * form like Evo 2's log_poles, as complex numbers:
 *   h[c, t] = Re sum_{n<N} R[c, n] exp(lam[c, n] t),   p = exp(lam),
 * where log_poles and residues are (D, N) complex, stored as (D, N, 2) fp32
 * (re, im) pairs; a pole p enters as lam = log|p| + i arg(p).  Modes with zero
 * imaginary parts give exactly the real-mode operator.  States are (B, D, N)
 * complex, stored as (B, D, N, 2) fp32 pairs.  Everything else -- layouts,
 * ownership, errors, workspace -- is as for the real-mode entry point of the
 * same name.
 */

/* h (D, L) fp32, as hyena_modal_filter. */
hyena_status_t hyena_modal_filter_cpx(const float* log_poles, const float* residues,
                                      int64_t D, int64_t N, int64_t L, float* h,
                                      hipStream_t stream);

/* Single pass, as hyena_fftconv_fwd (same workspace size). */
hyena_status_t hyena_fftconv_fwd_cpx(const void* x1, const void* x2, const void* v,
                                     const float* log_poles, const float* residues,
                                     int64_t N, const float* skip, void* y,
                                     int64_t B, int64_t D, int64_t L, hyena_dtype_t io,
                                     void* workspace, size_t ws_bytes, hipStream_t stream);

/* Chunked prefill with the complex modal state carried in and out, as
 * hyena_chunk_fwd:
 *   z[t] = sum_{k=t0}^{t} h[t-k] u[k] + Re sum_n R_n p_n^(t-t0+1) s_n,
 *   s_n <- p_n^C' s_n + sum_j p_n^(C'-1-j) u[t0+j].
 * The algorithm is AUTO: the matrix cores for N <= 16 complex modes (each a
 * pair of real lanes of its scan), per-chunk FFTs otherwise. */
hyena_status_t hyena_chunk_fwd_cpx(const void* x1, const void* x2, const void* v,
                                   const float* log_poles, const float* residues,
                                   int64_t N, const float* skip,
                                   const float* state_in, float* state_out,
                                   void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                                   hyena_dtype_t io, hipStream_t stream);

/* hyena_chunk_fwd_cpx with the algorithm chosen by the caller:
 * HYENA_CHUNK_MFMA takes N <= 16 complex modes, HYENA_CHUNK_FFT any N with
 * C' <= HYENA_MAX_FFT_CHUNK, AUTO as hyena_chunk_fwd_cpx. */
hyena_status_t hyena_chunk_fwd_cpx_algo(const void* x1, const void* x2, const void* v,
                                        const float* log_poles, const float* residues,
                                        int64_t N, const float* skip,
                                        const float* state_in, float* state_out,
                                        void* y, int64_t B, int64_t D, int64_t L, int64_t C,
                                        hyena_dtype_t io, hyena_chunk_algo_t algo,
                                        hipStream_t stream);

/* One decode step, as hyena_modal_decode: s_n <- p_n s_n + u,
 * y = x2 * Re sum_n R_n s_n + skip * u. */
hyena_status_t hyena_modal_decode_cpx(const void* x1, const void* x2, const void* v,
                                      const float* log_poles, const float* residues,
                                      int64_t N, const float* skip,
                                      const float* state_in, float* state_out,
                                      void* y, int64_t B, int64_t D, hyena_dtype_t io,
                                      hipStream_t stream);

/*
 * hyena_chunk_fwd_tokmajor -- the modal operator on the token-major layout
 * of the mixer's projections, with the state carried in and out.
 * in_proj's 3H output holds every channel's three streams side by side
 * (Hyena channels are interleaved per triple: evo2_flash README,
 * Limitations), and y feeds out_proj token by token (evo2_flash README,
 * layer_names table: 'blocks.N.projections', 'blocks.N.filter').  This entry
 * reads and writes those layouts directly, with no transposing pass:
 *   xin : (B, L, 3D) `io`; channel c's x1, x2 and v at columns
 *         3c + pos_x1, 3c + pos_x2 and 3c + pos_v, where (pos_x1, pos_x2,
 *         pos_v) is a permutation of (0, 1, 2) (the pages do not give the
 *         order within a triple, so the caller states it)
 *   y   : (B, L, D) `io`, written
 *   log_poles, residues : (D, N) fp32, 1 <= N <= HYENA_MAX_MODES
 *   skip : (D) fp32 or NULL
 *   state_in  : (B, D, N) fp32 or NULL (zero state)
 *   state_out : (B, D, N) fp32, written (may equal state_in)
 *   workspace : device buffer of at least hyena_chunk_tokmajor_workspace_size()
 *               bytes, 16-byte aligned, contents scratch (NULL when that size
 *               is 0); calls sharing one workspace must be ordered.
 * The result is that of hyena_chunk_fwd on the same streams, for any C:
 *   y[b, t, c] = x2 * (sum_{k<=t} h[c, t-k] u[k] + sum_n R_n p_n^(t+1) s_in_n)
 *                + skip[c] * u[t],  u = x1 * v.
 * Two evaluations (AUTO picks one by shape; hyena_chunk_fwd_tokmajor_algo
 * names one):
 *   HYENA_CHUNK_MFMA: the matrix-core chunk evaluation of hyena_chunk_fwd,
 *     one pass over blocks of 8 channels, inputs read once and y written
 *     once; bf16 with N <= 16, D a multiple of 8 below 349526, xin and y
 *     16-byte aligned (else HYENA_ERR_UNSUPPORTED); the workspace is not
 *     used and may be NULL.
 *   HYENA_CHUNK_RECURRENCE: per token with the decode step's recurrence
 *     s_n <- p_n s_n + u, over segments of the sequence that run in
 *     parallel: each segment's end state from zero, a scan of those over the
 *     segments, then every segment from its true entering state.
 * AUTO takes MFMA where it applies and the shape is at most 32 tiles of 1024
 * tokens per CU on at least 256 blocks of 8 channels (B D / 8 >= 256 and
 * B (D / 8) ceil(L / 1024) <= 8192), RECURRENCE otherwise.  B <= 65535.
 * L = 0 copies state_in to state_out.  Workspace NULL, short or misaligned
 * when one is needed -> HYENA_ERR_WORKSPACE.
 */
hyena_status_t hyena_chunk_fwd_tokmajor(const void* xin, int32_t pos_x1, int32_t pos_x2,
                                        int32_t pos_v, const float* log_poles,
                                        const float* residues, int64_t N, const float* skip,
                                        const float* state_in, float* state_out, void* y,
                                        int64_t B, int64_t D, int64_t L, hyena_dtype_t io,
                                        void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * hyena_fir_fwd_tokmajor -- the explicit-FIR operator (hcm K = 128, hcs
 * K = 7: Evo2-7B-262K model card, Implementation Notes, 'Block dispatch') on
 * the same token-major layout, continuing from a window like
 * hyena_fir_fwd_window.  With e = [window_in, u[0:L)], u = x1 * v:
 *   y[b, t, c] = x2 * sum_{k<K} taps[c, k] e[K-1+t-k] + skip[c] * u[t],
 * and window_out = the last K-1 entries of e (the FIR part of the inference
 * cache: Evo2-7B-262K model card, Implementation Notes, 'Custom cache').
 *   xin, pos_x1, pos_x2, pos_v, y, B, D, L, io : as hyena_chunk_fwd_tokmajor
 *   taps : (D, K) fp32, 1 <= K <= HYENA_MAX_FIR_TAPS_TOKMAJOR;  skip : (D) or NULL
 *   window_in  : (B, D, K-1) fp32, oldest first, or NULL (fresh sequence)
 *   window_out : (B, D, K-1) fp32, written (may equal window_in), or NULL
 *                (not kept)
 * Any L >= 0 (L = 1 per decode step); L = 0 moves the window.  Segments of
 * the sequence run in parallel, each reading K-1 tokens before it again.
 */
hyena_status_t hyena_fir_fwd_tokmajor(const void* xin, int32_t pos_x1, int32_t pos_x2,
                                      int32_t pos_v, const float* taps, int64_t K,
                                      const float* skip, const float* window_in,
                                      float* window_out, void* y, int64_t B, int64_t D, int64_t L,
                                      hyena_dtype_t io, hipStream_t stream);

/* hyena_chunk_fwd_tokmajor with the evaluation named: HYENA_CHUNK_AUTO,
 * HYENA_CHUNK_MFMA or HYENA_CHUNK_RECURRENCE (HYENA_CHUNK_FFT ->
 * HYENA_ERR_UNSUPPORTED, any other value -> HYENA_ERR_INVALID_ARG). */
hyena_status_t hyena_chunk_fwd_tokmajor_algo(const void* xin, int32_t pos_x1, int32_t pos_x2,
                                             int32_t pos_v, const float* log_poles,
                                             const float* residues, int64_t N,
                                             const float* skip, const float* state_in,
                                             float* state_out, void* y, int64_t B, int64_t D,
                                             int64_t L, hyena_dtype_t io, hyena_chunk_algo_t algo,
                                             void* workspace, size_t ws_bytes,
                                             hipStream_t stream);

/* Workspace bytes hyena_chunk_fwd_tokmajor needs for this shape on the
 * per-token path: B * P * D * N floats for its P segments, 0 when the sequence
 * is one segment or the shape is empty or unsupported.  (The matrix-core path
 * needs none; the size covers either, as the alignment of the buffers is not
 * known here.) */
size_t hyena_chunk_tokmajor_workspace_size(int64_t B, int64_t D, int64_t L, int64_t N,
                                           hyena_dtype_t io);

#ifdef __cplusplus
}
#endif

#endif /* HYENA_H_ */
