/*
 * sm_softmax.h -- C ABI of the MI355X (gfx950) fused row-softmax library (forward,
 * backward), the fused residual RMSNorm on the same row layout, and the fused
 * attention forward that carries the online softmax into QK^T and PV.
 *
 * Operation (every entry point below computes exactly this):
 *
 *     y[i,j] = exp(x[i,j] - m_i) / sum_k exp(x[i,k] - m_i),   m_i = max_k x[i,k]
 *
 * over an M x N matrix, softmax along the last dimension. This is the fused
 * softmax of "Triton: Writing GPU Kernels in Python, Measured" (section "Step 2:
 * a fused softmax") and of "Fused Softmax on GPU: From Naive PyTorch to
 * Persistent Triton Kernels" (section "Triton -- One Block Per Row", whose
 * kernel takes explicit input and output row strides). As in the Warpline
 * README's description of its softmax kernel, the reduction state (maximum and
 * sum) is FP32, irregular widths are masked, and the result is rounded once to
 * the storage dtype (round to nearest, ties to even).
 *
 * Layout: row i of the input starts at in + i*in_stride elements, row i of the
 * output at out + i*out_stride elements; columns are contiguous (stride 1).
 * Input and output share one dtype. Strides are in elements, not bytes.
 *
 * Ownership: `in` and `out` are device pointers on the current HIP device,
 * owned by the caller (hipMalloc, a torch tensor, ...). The library keeps only
 * a per-device cache of device properties and kernel occupancy. All launches
 * are asynchronous on `stream`; faults inside a kernel surface at the caller's
 * next synchronisation.
 *
 * Special values (readings where the pages say nothing, kept by every plan):
 *   - -inf entries give exactly 0; a row whose entries are all -inf gives a
 *     row of zeros (the pages' online-merge guard gives such a part a zero
 *     sum; this library then outputs 0 instead of 0/0);
 *   - a row holding NaN or +inf gives a row of NaN.
 *
 * Errors: every argument check runs on the host before any HIP call, so a
 * rejected call has no side effect. A zero-sized problem (M == 0 or N == 0)
 * returns SM_OK without launching anything and without touching the pointers.
 */
#ifndef SM_SOFTMAX_H
#define SM_SOFTMAX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SM_SOFTMAX_VERSION 10200 /* 1.2.0 */

typedef enum sm_dtype { SM_F32 = 0, SM_F16 = 1, SM_BF16 = 2 } sm_dtype;

typedef enum sm_status {
    SM_OK = 0,
    SM_ERR_INVALID = -1,   /* bad size, stride, pointer or alignment */
    SM_ERR_DTYPE = -2,     /* unknown dtype code */
    SM_ERR_OVERLAP = -3,   /* out overlaps in other than exactly in place */
    SM_ERR_HIP = -4,       /* a HIP runtime call or kernel launch failed */
    SM_ERR_NO_DEVICE = -5, /* no usable HIP device */
    SM_ERR_WORKSPACE = -6, /* caller workspace too small or misaligned */
    SM_ERR_PLAN = -7       /* forced plan or shape cannot cover this problem */
} sm_status;

/* Plans: the three kernel paths.
 *   RESIDENT   -- one-pass; every row is held in registers by one group of
 *                 lanes (a sub-wave, a wave, or a workgroup of up to 16 waves
 *                 with a cross-wave step in LDS); the grid covers every row
 *                 once. Each element is read once and written once.
 *   PERSISTENT -- the same one-pass row body, launched on occupancy x CUs
 *                 workgroups that walk the rows with a grid stride and load
 *                 the next row while computing the current one ("Fused
 *                 Softmax on GPU", section "Persistent Triton Kernel").
 *   WIDE       -- rows too wide to hold: pass 1 runs the online (max, sum)
 *                 recurrence over 1024-element chunks and writes one FP32
 *                 (max, sum) pair per wave; pass 2 merges a row's pairs and
 *                 re-reads the row to normalise and write ("Measured
 *                 optimization case studies", section "Wide rows: loop in one
 *                 program, or split across programs"; Warpline README, the
 *                 description of its online path).
 *   SPLIT      -- rows too wide to hold in one workgroup, in one launch: a row
 *                 is cut into P slices of 256 * V 16-byte windows, one 256-lane
 *                 workgroup holds a slice in registers, publishes its slice's
 *                 (max, sum) pair, waits (bounded) for the row's other slices,
 *                 merges the P pairs in a fixed order and writes its slice.
 *                 Each element is read once and written once. The grid is a
 *                 multiple of P and at most half of the resident capacity
 *                 (further rows are taken in rounds), so a row's slices are
 *                 resident together unless the device is filled by other
 *                 work; more than two SPLIT calls running at once on different
 *                 streams of one device can exceed it. Every wait is bounded
 *                 (spin_limit polls), so every call ends. A wait that runs out
 *                 is counted (sm_softmax_sync_failures); out of place, its
 *                 workgroup then reads the whole input row for the row's
 *                 maximum and sum itself, so the output is the softmax whatever
 *                 the scheduling; in place (out == in), where the row's other
 *                 slices may already have overwritten their input, it writes
 *                 NaN over its slice.
 * Graph capture: a SPLIT call tags its exchange with an id fixed at launch, which
 * a graph would replay unchanged. On a stream that is capturing, AUTO therefore
 * takes WIDE where it would take SPLIT, and a forced SPLIT returns SM_ERR_PLAN
 * (the same holds for the backward; the RMSNorm call takes its two-launch form).
 * sm_softmax_plan_query reports the plan of a call on a stream that is not
 * capturing.
 * AUTO runs a row one-pass when N <= 8192, or when the row fits in 4096
 * 16-byte windows (8192 for FP32 forward rows) and there are at least 128 rows;
 * otherwise it takes SPLIT when a row's slices fit the resident capacity, WIDE
 * when they do not (and, for FP32 forward rows of at least 2^17 windows, WIDE
 * when SPLIT would need four or more rounds). A one-pass row is held in the
 * narrowest measured-best group (16 to 1024 lanes, 1 to 8 vectors per lane),
 * PERSISTENT when the row groups fit in at most two rounds of resident
 * workgroups, RESIDENT when there are more. */
typedef enum sm_plan {
    SM_PLAN_AUTO = 0,
    SM_PLAN_RESIDENT = 1,
    SM_PLAN_PERSISTENT = 2,
    SM_PLAN_WIDE = 3,
    SM_PLAN_SPLIT = 4
} sm_plan;

/* Optional launch overrides (zero-initialise for "automatic"). */
typedef struct sm_softmax_opts {
    int plan;            /* sm_plan */
    int lanes_per_row;   /* RESIDENT/PERSISTENT: 16, 32, 64, 128, 256, 512 or 1024; 0 = auto */
    int vecs_per_lane;   /* RESIDENT/PERSISTENT/SPLIT: 16-byte vectors per lane, 1, 2, 4 or 8
                            (backward: at most 4); 0 = auto */
    int grid;            /* workgroups to launch; 0 = auto (SPLIT: a multiple of the
                            slices per row, at most half the resident capacity) */
    int chunks_per_wave; /* WIDE: 1024-element chunks per wave; 0 = auto */
    int prefetch;        /* PERSISTENT: 1 = load the next row early, -1 = no; 0 = auto */
    int nontemporal;     /* streaming (nontemporal) loads of the input: 1 = yes, -1 = no,
                            0 = auto: yes when the call moves at least 1 GiB (four times
                            the MI355X MALL) in the forward and in SPLIT and WIDE plans,
                            32 MiB in one-pass backward rows, 256 MiB in one-pass RMSNorm
                            rows; one-pass plans have them on 128- to 1024-lane rows
                            without prefetch, the WIDE plan on both passes */
    int spin_limit;      /* SPLIT: polls a workgroup may spend waiting for the other
                            slices of a row; 0 = default (2^20, about a second) */
    /* Optional timing events (created by the caller with hipEventCreate), or NULL.
     * They are attached to the kernel dispatches themselves (hipExtLaunchKernel):
     * start_event takes the start time of the call's first kernel and stop_event
     * the end time of its last, so their elapsed time is the device time of the
     * call without host-side launch latency. */
    hipEvent_t start_event;
    hipEvent_t stop_event;
} sm_softmax_opts;

/* What a call would launch (filled by sm_softmax_plan_query). */
typedef struct sm_plan_info {
    int plan;              /* resolved sm_plan (never AUTO) */
    int lanes_per_row;
    int vecs_per_lane;
    int prefetch;
    int nt_loads;          /* 1 = streaming (nontemporal) loads */
    int block;             /* threads per workgroup */
    int64_t grid;          /* workgroups per launch */
    int chunks_per_wave;   /* WIDE only */
    int64_t waves_per_row; /* WIDE: waves per row; SPLIT: slices (workgroups) per row */
    int launches;          /* 1, or 2 for WIDE */
    int same_phase;        /* input and output rows share their 16-byte phase */
    int64_t workspace_bytes; /* WIDE scratch: M * waves_per_row * 8 bytes;
                                SPLIT: M * slices per row * 32 bytes (both rounded up
                                to 256) */
    int64_t model_bytes;   /* algorithmic bytes: 2*M*N*elem one-pass and SPLIT, 3*M*N*elem
                              WIDE (backward: 3*M*N*elem one-pass and SPLIT, 5*M*N*elem
                              WIDE) */
    int dy_same_phase;     /* backward: dy rows share y's 16-byte phase (vector loads) */
    int slice_windows;     /* SPLIT: 16-byte windows per slice (a row's windows spread
                              evenly over its slices; at most 256 * vecs_per_lane) */
} sm_plan_info;

/*
 * Fused row softmax, asynchronous on `stream` (0 = the null stream).
 *   in, out     : device pointers, element-aligned; out == in with
 *                 out_stride == in_stride is allowed (in place); any other
 *                 overlap of the two row sets -> SM_ERR_OVERLAP
 *   M, N        : rows and columns (N <= 2^31 - 1)
 *   in_stride,
 *   out_stride  : row strides in elements, >= N when M > 1
 *   dtype       : sm_dtype of both tensors
 * The WIDE and SPLIT plans take their scratch from a buffer the library keeps per
 * (device, stream): allocated (hipMalloc) by the first call on the stream that needs
 * scratch, replaced by a larger one (at least twice the size) when a call needs more,
 * and held, with any buffer it replaced, until the process ends (32 bytes per SPLIT
 * slice, 8 per WIDE wave: 32 KiB for 64 x 131072 BF16 rows; at least 64 KiB is
 * allocated). Calls on one stream run in order and share it; calls on different streams
 * never do. On a stream that is capturing a graph the scratch comes from hipMallocAsync
 * instead (a graph memory node, freed within the graph). The first SPLIT call on a
 * stream also allocates that stream's failure counter (hipMalloc + hipMemset of 256
 * bytes, kept until the process ends). sm_softmax_fwd_noalloc allocates nothing.
 * Returns SM_OK or a negative sm_status.
 */
int sm_softmax_fwd(const void *in, void *out, int64_t M, int64_t N, int64_t in_stride,
                   int64_t out_stride, int dtype, hipStream_t stream);

/*
 * As sm_softmax_fwd, with launch overrides and optional caller scratch.
 *   opts        : NULL = automatic
 *   workspace   : device memory of at least plan_info.workspace_bytes, 16-byte
 *                 aligned, used only by the WIDE and SPLIT plans; NULL = the
 *                 library's per-stream buffer, as sm_softmax_fwd. The caller must not
 *                 reuse it until the call's work on `stream` has finished.
 */
int sm_softmax_fwd_ex(const void *in, void *out, int64_t M, int64_t N, int64_t in_stride,
                      int64_t out_stride, int dtype, const sm_softmax_opts *opts,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory -- code under graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: sm_softmax_fwd with the same
 * arguments and result, making no allocation (no hipMalloc, hipFree or stream-ordered
 * pool call). The WIDE and SPLIT plans take their scratch, and SPLIT its failure
 * counter, from one array of the library's own per device (SM_NOALLOC_SCRATCH_BYTES
 * of workspace plus 256 bytes, held until the process ends). A problem whose plan
 * needs more than SM_NOALLOC_SCRATCH_BYTES of workspace (plan_info.workspace_bytes
 * of sm_softmax_plan_query) returns SM_ERR_WORKSPACE before launching anything; one-
 * pass plans need none. Every call on a device shares that device's array, so calls
 * that overlap in time on one device (different streams, or host threads) race on it
 * and must be ordered by the caller. SPLIT waits that run out re-read their input row
 * (out of place) and are not reported; calls in place take WIDE where AUTO would take
 * SPLIT, as do calls on a capturing stream, so no result depends on scheduling.
 * Returns SM_OK or a negative sm_status.
 */
#define SM_NOALLOC_SCRATCH_BYTES (1u << 20)
int sm_softmax_fwd_noalloc(const void *in, void *out, int64_t M, int64_t N, int64_t in_stride,
                           int64_t out_stride, int dtype, hipStream_t stream);

/*
 * Resolve the plan a call would use, without launching anything.
 *   num_cus > 0 : evaluate on the host only for a device with that many
 *                 compute units (occupancy assumed: 8 workgroups of 256
 *                 threads per CU); no HIP call is made
 *   num_cus == 0: use the current HIP device and its measured occupancy
 * Pointers are used only for their alignment and overlap.
 */
int sm_softmax_plan_query(const void *in, const void *out, int64_t M, int64_t N,
                          int64_t in_stride, int64_t out_stride, int dtype,
                          const sm_softmax_opts *opts, int num_cus, sm_plan_info *info);

/*
 * Softmax backward: dx = y * (dy - sum_j y_j * dy_j) per row, where y is the
 * softmax output saved by the forward call and dy the gradient of the loss with
 * respect to y ("Measured optimization case studies", section "Training:
 * backward kernels through autograd"). FP32 dot product (compensated, with exact
 * products, for FP32 data), one rounding of dx to the storage dtype.
 *   y, dy, dx   : device pointers of one dtype, element-aligned; dx may be y or
 *                 dy exactly (same pointer and stride: in place); any other
 *                 overlap of dx with y or dy -> SM_ERR_OVERLAP (y and dy may
 *                 overlap each other: both are only read)
 *   strides     : row strides in elements, >= N when M > 1
 * Plans as for the forward call: one-pass RESIDENT/PERSISTENT for N <= 8192, and
 * for rows of up to 4096 16-byte windows when there are at least 128 of them
 * (3*M*N*elem bytes); other rows SPLIT (one launch, the slices' partial dots
 * exchanged as the forward exchanges its (max, sum) pairs: 3*M*N*elem bytes; a
 * wait that runs out is counted, and its workgroup then re-reads the row's y and
 * dy for the dot when dx aliases neither, or writes NaN over its slice), or WIDE
 * where a row's slices cannot be resident together or the stream is capturing a
 * graph (two passes, a partial dot per wave, then merge and apply: 5*M*N*elem
 * bytes). SPLIT and WIDE take their scratch (M * slices * 32 or M * waves_per_row
 * * 8 bytes) from the library's per-stream buffer, as the forward, or caller
 * workspace through the _ex form.
 * Returns SM_OK or a negative sm_status; validation as for sm_softmax_fwd.
 */
int sm_softmax_bwd(const void *y, const void *dy, void *dx, int64_t M, int64_t N,
                   int64_t y_stride, int64_t dy_stride, int64_t dx_stride, int dtype,
                   hipStream_t stream);

/* As sm_softmax_bwd with overrides (plan, lanes_per_row, vecs_per_lane in {1, 2, 4},
 * grid, chunks_per_wave, nontemporal (one-pass rows of 128 to 1024 lanes), timing
 * events) and optional caller workspace. Automatic one-pass plans launch one
 * workgroup per row group (RESIDENT); PERSISTENT is available when forced. */
int sm_softmax_bwd_ex(const void *y, const void *dy, void *dx, int64_t M, int64_t N,
                      int64_t y_stride, int64_t dy_stride, int64_t dx_stride, int dtype,
                      const sm_softmax_opts *opts, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* The plan sm_softmax_bwd would launch (num_cus as for sm_softmax_plan_query). */
int sm_softmax_bwd_plan_query(const void *y, const void *dy, const void *dx, int64_t M, int64_t N,
                              int64_t y_stride, int64_t dy_stride, int64_t dx_stride, int dtype,
                              const sm_softmax_opts *opts, int num_cus, sm_plan_info *info);

/*
 * Fused residual RMSNorm on the same row layout (Warpline README, the description
 * of its K1 kernel: the input and residual are added in FP32 and that sum is
 * rounded once to the input dtype; the RMS reduction runs in FP32; the weight is
 * applied and the result rounded once to the input dtype). Per row i:
 *
 *     s_j = rn_dtype(x_ij + r_ij)             (s_j = x_ij without a residual)
 *     y_ij = rn_dtype(s_j * w_j / sqrt(sum_k s_k^2 / N + eps))
 *
 *   x, residual  : device pointers of one dtype; residual may be NULL
 *   weight       : N elements of the same dtype, shared by every row (must not
 *                  overlap y or residual_out)
 *   y            : output; may be x or residual exactly (same pointer and stride)
 *   residual_out : optional (NULL): receives s, the rounded sum (the residual
 *                  stream of the next layer); may be x or residual exactly, must
 *                  not overlap y
 *   strides      : row strides in elements, >= N when M > 1
 *   eps          : finite, >= 0 (the pages give no value; 0 lets a zero row give NaN)
 * Reduction state is FP32: rows whose sum of squares exceeds the FP32 range give
 * zeros (or NaN where s is infinite). Plans as for the softmax backward: one-pass
 * RESIDENT/PERSISTENT rows (up to 4 vectors per lane), SPLIT for wide rows (one
 * launch, partial sums of squares exchanged between the row's workgroups), and
 * WIDE as two launches of the split kernel (publish, then gather and apply) when
 * a row's slices cannot be resident together, when rows need more than 64
 * slices and several rounds (measured faster), or on a stream that is capturing a
 * graph. A SPLIT wait that runs out is counted as for the softmax; the workgroup
 * then re-reads its row's x (and residual) for the sum of squares when neither y
 * nor residual_out aliases x or the residual, and writes NaN over its slice
 * otherwise. model_bytes counts the compulsory HBM bytes: x, y and, when present,
 * the residual and residual_out once per element, w once (N elements); WIDE reads x
 * and the residual twice. (The pages' requested-
 * byte convention counts w once per row in addition.)
 * Returns SM_OK or a negative sm_status; validation as for sm_softmax_fwd.
 */
int sm_rmsnorm_fwd(const void *x, const void *residual, const void *weight, void *y,
                   void *residual_out, int64_t M, int64_t N, int64_t x_stride, int64_t res_stride,
                   int64_t y_stride, int64_t res_out_stride, float eps, int dtype,
                   hipStream_t stream);

/* As sm_rmsnorm_fwd with overrides (plan, lanes_per_row, vecs_per_lane in {1, 2, 4},
 * grid, nontemporal, spin_limit, timing events) and optional caller workspace. */
int sm_rmsnorm_fwd_ex(const void *x, const void *residual, const void *weight, void *y,
                      void *residual_out, int64_t M, int64_t N, int64_t x_stride,
                      int64_t res_stride, int64_t y_stride, int64_t res_out_stride, float eps,
                      int dtype, const sm_softmax_opts *opts, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* The plan sm_rmsnorm_fwd would launch (num_cus as for sm_softmax_plan_query). */
int sm_rmsnorm_plan_query(const void *x, const void *residual, const void *weight, const void *y,
                          const void *residual_out, int64_t M, int64_t N, int64_t x_stride,
                          int64_t res_stride, int64_t y_stride, int64_t res_out_stride, float eps,
                          int dtype, const sm_softmax_opts *opts, int num_cus,
                          sm_plan_info *info);

/*
 * Fused attention forward with the online softmax (the step after the row softmax
 * that "Fused Softmax on GPU" names in its closing section: fusing the online
 * softmax with the matmul before it, as FlashAttention does). For each of BH heads
 * and query row i, without writing the scores:
 *
 *     S_ij = scale * q_i . k_j     (masked to -inf for j > i + Sk - Sq when causal)
 *     o_i  = sum_j softmax(S_i)_j v_j,   lse_i = log sum_j exp(S_ij)
 *
 *   q [BH][Sq][d], k and v [BH][Sk][d], o [BH][Sq][d]: device pointers, FP16 or BF16,
 *     element (h, i, c) at base + h * head_stride + i * row_stride + c (elements);
 *     bases 16-byte aligned, strides multiples of 8 elements, d <= row strides <=
 *     2^24; the heads of o must not share elements; o must not overlap q, k, v or lse
 *   lse  : optional (NULL) FP32 [BH][Sq] contiguous; -inf for a query that sees no key
 *   d    : 64 or 128
 *   scale: finite (usually 1 / sqrt(d)); causal: 0 or 1 (the mask is aligned to the
 *          bottom right, so the last query sees every key)
 * Scores and statistics are FP32; the probabilities are rounded to the input dtype
 * before the product with V (the FlashAttention contract); o is rounded once. A
 * query that sees no key gives zeros (the all -inf row reading of the softmax).
 * Workgroups of 4 waves own 128 query rows of one head (causal: two such q-blocks,
 * i and n-1-i, so every workgroup does about the same work) and walk the keys in
 * blocks of 64 through LDS; products run on v_mfma_f32_16x16x32. The result does not
 * depend on the grid order: repeated calls give identical bits.
 * Returns SM_OK or a negative sm_status (SM_ERR_DTYPE for FP32).
 */
int sm_attention_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t BH,
                     int64_t Sq, int64_t Sk, int64_t d, int64_t q_row_stride,
                     int64_t q_head_stride, int64_t k_row_stride, int64_t k_head_stride,
                     int64_t v_row_stride, int64_t v_head_stride, int64_t o_row_stride,
                     int64_t o_head_stride, float scale, int causal, int dtype, hipStream_t stream);

/* As sm_attention_fwd; opts supplies only the timing events (other fields ignored). */
int sm_attention_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t BH, int64_t Sq, int64_t Sk, int64_t d, int64_t q_row_stride,
                        int64_t q_head_stride, int64_t k_row_stride, int64_t k_head_stride,
                        int64_t v_row_stride, int64_t v_head_stride, int64_t o_row_stride,
                        int64_t o_head_stride, float scale, int causal, int dtype,
                        const sm_softmax_opts *opts, hipStream_t stream);

/* Static text for a status code. */
const char *sm_softmax_strerror(int status);

/* SM_SOFTMAX_VERSION of the built library. */
int sm_softmax_version(void);

/* The hipError_t of the most recent SM_ERR_HIP on the calling thread (0 if none). */
int sm_softmax_last_hip_error(void);

/*
 * SPLIT-plan waits that ran out of polls on `stream` since its counter was
 * created (each one re-read its whole input row, or, in place, wrote NaN over
 * its row slice). Synchronises `stream`, then reads the count into *count (0 if
 * no SPLIT call ran on that stream).
 * Returns SM_OK, SM_ERR_INVALID for a NULL count, or SM_ERR_HIP.
 */
int sm_softmax_sync_failures(hipStream_t stream, unsigned int *count);

#ifdef __cplusplus
}
#endif

#endif /* SM_SOFTMAX_H */
