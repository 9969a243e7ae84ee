/*
 * pa.h -- C ABI of the packed-AdamW step library (libpa.so, gfx950).
 *
 * One optimizer update of AdamW whose two moments persist, between updates,
 * in a compact form, with the current update itself done in FP32:
 *
 *   m' = beta1*m + (1-beta1)*g
 *   v' = beta2*v + (1-beta2)*g*g
 *   p' = p*(1-lr*wd) - (lr/(1-beta1^t)) * m' / (sqrt(v'/(1-beta2^t)) + eps)
 *
 * (TurboAdam package page, "The AdamW update remains AdamW": the recurrence
 * and the decoupled-decay update; KBench quantized-optimizer-state
 * reference, `quantized_adamw_step`: the FP32 operation order used here,
 * left to right, with the host scalars formed in double precision and each
 * rounded once to binary32.)
 *
 * Modes (Packed AdamW Reference README, introduction; its project page,
 * Release scope):
 *   PA_PACKED_E4   one uint32 per parameter: low 16 bits a signed finite
 *                  E4M11 first moment, high 16 bits an unsigned finite E4M12
 *                  uncorrected RMS (sqrt of the second moment).  The prior
 *                  word is decoded, v = r*r, the update runs in FP32 on the
 *                  new unquantised moments, and only then m' and sqrt(v')
 *                  are rounded to nearest (ties to even) with saturation at
 *                  the largest finite value and packed.  Exponent bias 15 in
 *                  both lanes, gradual underflow, no Inf/NaN codes; NaN packs
 *                  as code 0.
 *   PA_PACKED_FP16 the same word with IEEE binary16 in both halves
 *                  (round to nearest even, overflow to Inf).
 *   PA_FP32        plain FP32 AdamW with two FP32 moment tensors.
 *   PA_BLOCKWISE8  8-bit codes for both moments, one FP32 absmax per
 *                  2048-element block per moment, ascending 256-entry code
 *                  maps, nearest-entry requantisation through the 255 FP32
 *                  midpoints (ties to the lower entry), BF16 parameter output
 *                  (KBench quantized-optimizer-state reference,
 *                  `quantized_adamw_step` and `_requantise`).
 *
 * Execution contract (project page, Execution contract table): contiguous
 * FP32 parameters and dense FP32 gradients on one device, one group of
 * hyperparameters and one global step per call.
 *
 * Memory: every pointer handed to pa_step / pa_step_list that names tensor
 * data is a DEVICE pointer owned by the caller; the library never frees or
 * keeps it beyond the call.  Descriptor structs (pa_hyper, pa_fp32_state,
 * pa_blockwise_state) and the pointer/size arrays of pa_step_list are HOST
 * memory, read during the call only.  State must be zero-filled by the
 * caller before step 1 (the all-zero word and a zero absmax both decode to
 * zero moments).
 *
 * Streams: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without waiting.  Faults inside a kernel
 * surface at the next synchronisation of that stream.
 *
 * Errors: every entry point returns PA_OK (0) or a negative PA_ERR_* code
 * and never aborts or throws.  A call that returns an error has enqueued
 * nothing.  There is no fallback to code off the GPU (no CPU or eager
 * path); the blockwise step's choice between its two GPU launches
 * (pa_step_list) gives the same results either way.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_FP32 = 0,
  PA_PACKED_E4 = 1,
  PA_PACKED_FP16 = 2,
  PA_BLOCKWISE8 = 3
} pa_mode;

/* Element types of parameters and gradients for the typed entry points.
 * The update always runs in FP32: 16-bit values widen exactly and the new
 * parameter is rounded back to its own type, to nearest even (Inf past the
 * largest finite value).  The KBench quantized-optimizer-state reference
 * widens its inputs with .float() and narrows its output to bfloat16; the
 * TurboAdam package page, Verification, runs fp16, bf16 and fp32
 * parameters. */
typedef enum {
  PA_DT_F32 = 0,
  PA_DT_BF16 = 1,
  PA_DT_F16 = 2
} pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_ARG = -1,    /* null pointer with n > 0, unknown mode, step < 1,
                         beta outside [0,1), non-finite or negative lr/eps/wd,
                         non-finite beta */
  PA_ERR_ALIGN = -2,  /* a data pointer not aligned to its element, or the
                         buffers of one tensor not at one position modulo
                         four elements (one 16-byte phase for FP32 data);
                         blockwise: params/grads not 16-byte aligned */
  PA_ERR_SHAPE = -3,  /* blockwise length not a multiple of 2048 */
  PA_ERR_ALIAS = -4,  /* two buffers of one call overlap */
  PA_ERR_DEVICE = -5, /* the HIP runtime refused a launch or a copy */
  PA_ERR_NOMEM = -6,  /* the launch plan table could not be allocated */
  PA_ERR_CAPACITY = -7 /* pa_step_list_noalloc: more non-empty tensors than
                          PA_NOALLOC_MAX_TENSORS */
};

/* Hyperparameters, host doubles (TurboAdam package page, API section: lr,
 * betas, eps, weight_decay).  `nonfinite`, if not NULL, is a device counter
 * that the call increments by the number of elements whose new parameter,
 * first moment or second moment is not finite (the optimizer non-finite
 * count of the reference's one-update smoke check).
 *
 * Two optional device inputs let a caller feed the gradient pre-pass
 * (pa_grad_stats_list) into the update without a host round trip:
 *   grad_scale       if not NULL, a device float read by the kernels: every
 *                    gradient, after widening to FP32, is multiplied by it
 *                    (one binary32 multiplication) before the update.  Used
 *                    for global-norm clipping; NULL leaves gradients as
 *                    they are (exactly as a scale of 1 would).
 *   skip_if_nonzero  if not NULL, a device counter read by the kernels:
 *                    when it is nonzero the call changes nothing (no
 *                    parameter, state or counter is written).  Used to skip
 *                    an update whose gradients hold NaN or Inf.
 * Both are read on `stream`, after the work enqueued before the call. */
typedef struct {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
  unsigned long long* nonfinite;
  const float* grad_scale;
  const unsigned long long* skip_if_nonzero;
} pa_hyper;

/* PA_FP32 state: two device arrays of n floats. */
typedef struct {
  float* m;
  float* v;
} pa_fp32_state;

/* PA_BLOCKWISE8 state.  m_code/v_code: n device bytes; m_absmax/v_absmax:
 * n/2048 device floats; qmap_m/qmap_v: 256 ascending device floats each
 * (read only); p_out_bf16: n device uint16 receiving the updated parameters
 * as bfloat16 bits.  In this mode `params` is read only. */
typedef struct {
  uint8_t* m_code;
  float* m_absmax;
  uint8_t* v_code;
  float* v_absmax;
  const float* qmap_m;
  const float* qmap_v;
  uint16_t* p_out_bf16;
} pa_blockwise_state;

/* One tensor of n parameters, updated in place, step t = `step` (>= 1,
 * counting this update): the update at the top of this file (KBench
 * quantized-optimizer-state reference, `quantized_adamw_step`: params,
 * grads, state, step and hyperparameters in, new params and state out; the
 * packed word of the Packed AdamW Reference README, introduction).
 *   PA_PACKED_E4 / PA_PACKED_FP16: `state` is a device uint32_t* of n words.
 *   PA_FP32:       `state` is a host pa_fp32_state*.
 *   PA_BLOCKWISE8: `state` is a host pa_blockwise_state*.
 * n == 0 enqueues nothing and returns PA_OK.  `stream` is a hipStream_t. */
int pa_step(int mode, float* params, const float* grads, void* state, size_t n,
            const pa_hyper* hyper, long long step, void* stream);

/* `count` tensors sharing one hyperparameter set and one step (project
 * page, Execution contract table: one parameter group, one global step;
 * the update of each element as for pa_step).  Elementwise modes: one
 * launch over a table of all of them, cut into 4096-element tiles (1024
 * for lists under 32 Mi elements), one workgroup per tile (a list of more
 * than 2^22 tiles takes one launch per 2^22).  Blockwise mode, per tensor: from 48 blocks per workgroup slot
 * up, two launches, one workgroup that builds the search tables of the
 * map pair into a device buffer the library keeps per device and stream,
 * then one workgroup per 12 consecutive blocks in dispatch order; smaller
 * tensors, every call under graph capture, and a stream whose buffer
 * cannot be allocated, one persistent launch whose workgroups build the
 * tables themselves; the results are the same.  params[i], grads[i],
 * states[i] and n[i] describe tensor i exactly as for pa_step.  The table is
 * uploaded once per distinct list of parameter and state pointers and sizes
 * and cached (see pa_release_plans); the gradients are not part of it:
 * when a call's gradients differ from those in the table (torch allocates
 * new ones after zero_grad(set_to_none=True)), they are checked as at the
 * table's creation and written into it by small kernels on `stream`, with
 * no allocation or synchronisation.  Tensors of length 0 are skipped.
 * Once a list's table exists, a call enqueues those small kernels (when
 * needed) and its launch and nothing else (no allocation, host copy,
 * memset or synchronisation), so it can be captured in a HIP graph; a
 * captured call keeps the step, scalars and gradients it was captured with
 * (a table that a graph holds gets its gradients written on every call).
 * Calls on one list from different streams must be ordered by the caller. */
int pa_step_list(int mode, size_t count, float* const* params, const float* const* grads,
                 void* const* states, const size_t* n, const pa_hyper* hyper, long long step,
                 void* stream);

/* pa_step / pa_step_list with 16-bit parameters and/or gradients.
 * Supported (param_dtype, grad_dtype) pairs: (F32, F32), (BF16, BF16),
 * (F16, F16), (BF16, F32), (F16, F32); any other pair is PA_ERR_ARG, and
 * so is a 16-bit type with PA_BLOCKWISE8.  `params` and `grads` point to n
 * device elements of their type (bfloat16 / binary16 as uint16 bit
 * patterns); state is as for pa_step.  Alignment: every buffer aligned to
 * its element size, and all buffers of a tensor at the same position modulo
 * four elements (PA_ERR_ALIGN otherwise).  pa_step and pa_step_list are the
 * (F32, F32) case. */
int pa_step_typed(int mode, int param_dtype, int grad_dtype, void* params, const void* grads, void* state,
                  size_t n, const pa_hyper* hyper, long long step, void* stream);

int pa_step_list_typed(int mode, int param_dtype, int grad_dtype, size_t count, void* const* params,
                       const void* const* grads, void* const* states, const size_t* n,
                       const pa_hyper* hyper, long long step, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * pa_step_list_typed with the same arguments, results and errors, except
 * that the tensor table lives in a static device array of the library
 * (one per GPU, held until the process ends) instead of a cached plan.
 * The call makes no hipMalloc, hipFree or other allocating device call: it
 * writes the list's table into that array with small kernels on `stream`
 * and then launches the step, every call (nothing is cached).  At most
 * PA_NOALLOC_MAX_TENSORS non-empty tensors per call (PA_ERR_CAPACITY
 * beyond, before anything is enqueued).  Every call on one GPU shares the
 * array: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race on it and may update the wrong
 * tensors; calls ordered on one stream are safe.  Blockwise mode takes the
 * persistent launch at every size (it needs no buffer) and gives the
 * results of pa_step_list_typed. */
#define PA_NOALLOC_MAX_TENSORS 4095
int pa_step_list_noalloc(int mode, int param_dtype, int grad_dtype, size_t count, void* const* params,
                         const void* const* grads, void* const* states, const size_t* n,
                         const pa_hyper* hyper, long long step, void* stream);

/* Gradient pre-pass over `count` gradient tensors of one element type
 * (PA_DT_F32, PA_DT_BF16 or PA_DT_F16; grads[i] points to n[i] device
 * elements), in one persistent launch and one read of every gradient,
 * followed by a one-workgroup finalizer.  Device outputs, overwritten:
 *   sumsq       (required) the sum of the squares of all gradients, in
 *               double: each square is exact in double and the partial sums
 *               follow a fixed order for a given device and list, so the
 *               result is reproducible; it differs from the exact sum by at
 *               most the rounding of a double summation (NaN if any
 *               gradient is NaN, else +Inf if any is infinite).
 *   nonfinite   (nullable) the number of NaN or infinite gradients.
 *   clip_scale  (nullable) min(1, max_norm / (sqrt(sumsq) + 1e-6)), formed
 *               in double and rounded once to binary32 (NaN stays NaN);
 *               requires a finite max_norm > 0.
 * Pass clip_scale as pa_hyper.grad_scale and nonfinite as
 * pa_hyper.skip_if_nonzero of the following update for clipping and an
 * overflow skip with no host synchronisation.  The pages train AdamW on
 * dense FP32, FP16 and BF16 gradients (TurboAdam package page,
 * Verification; KBench reference, `grads.float()`) and gate on a non-finite
 * optimizer count (Packed AdamW Reference README, One-update smoke test).
 * Gradients must be aligned to their element size and must not overlap the
 * outputs.  The tensor table and per-workgroup partials are cached per
 * distinct list of lengths and gradient phases (address in elements modulo
 * 4) and stream, with the gradient pointers written into the table as for
 * pa_step_list (see pa_release_plans): calls on different streams use
 * separate partials; two calls on one stream are ordered by it.  count == 0,
 * or only empty tensors, writes 0, 0 and the coefficient of a zero norm. */
int pa_grad_stats_list(int grad_dtype, size_t count, const void* const* grads, const size_t* n,
                       double max_norm, double* sumsq, unsigned long long* nonfinite, float* clip_scale,
                       void* stream);

/* ------------------------------------------------------------------------
 * TurboAdam compressed state (TurboAdam package page, "How it works": UState
 * for the first moment, 1Q for the second, "Fused CUDA path").  The update
 * itself is the FP32 AdamW step above, on moments decoded from the state;
 * afterwards the second moment is re-encoded with 1Q and the first moment,
 * in normalised update units q = (m/bc1) / (sqrt(v_persisted/bc2) + eps),
 * with UState.  Readings of what the page leaves open (code levels, grid,
 * scale rule, random draws) are stated in adamw_step_amd/csrc/turbo.hpp.
 *
 * Layout (TurboAdam package page, "Fused CUDA path" and API: block_size,
 * m_block_size, v_bits): a 1Q block of B values (a power of two from 32 to
 * 1024, default 128) shares one pair of log2 endpoints; a UState group of G
 * values (a power of two dividing B, default 64) shares one mean; indices
 * have 2, 3, 4, 6 or 8 bits (default 4), packed densely: value i occupies
 * bits [v_bits*i, v_bits*i + v_bits) of the little-endian bit stream of
 * 32-bit words, so 3- and 6-bit indices straddle words.
 *
 * Per tensor, device buffers (all caller-owned, zero-filled before step 1):
 *   compress_m != 0 (UState): m_codes 4*ceil(n/16) bytes of 2-bit codes,
 *     m_means ceil(n/G) bfloat16, scalars 3 floats (decode scale, encode
 *     scale, accumulator); else m_fp32, n floats.
 *   compress_v != 0 (1Q): v_index 4*ceil(n*v_bits/32) bytes of indices,
 *     v_ends 2*ceil(n/B) binary16 (low, high log2 endpoint per block);
 *     else v_fp32, n floats.
 *   tensor_id keys the tensor's counter-based random draws (keep it fixed
 *   across steps and distinct across tensors).
 * Parameters and gradients are FP32, 16-byte aligned (pa_turbo_step_list_typed
 * also takes 16-bit ones, 8-byte aligned); m_fp32/v_fp32 16-byte,
 * m_codes/v_index/v_ends/scalars 4-byte, m_means 2-byte aligned
 * (PA_ERR_ALIGN otherwise).  With compress_m the page requires
 * beta1^2 < beta2 (PA_ERR_ARG otherwise).  The draws' counter holds the
 * value index / 4 and the step in 32 bits each, so a tensor holds at most
 * 2^34 values (PA_ERR_ARG beyond). */
typedef struct {
  int compress_m;
  int compress_v;
  uint32_t tensor_id;
  uint8_t* m_codes;
  uint16_t* m_means;
  float* m_fp32;
  uint8_t* v_index;
  uint16_t* v_ends;
  float* v_fp32;
  float* scalars;
} pa_turbo_state;

/* v_bits: 1Q index width, 2, 3, 4 (the page's default), 6 or 8.
 * m_step_factor: the UState scale factor (the page's default 1.1).  seed:
 * the rounding seed (the page's default 0x12345678).  block_size,
 * m_block_size: B and G above, 0 for the defaults 128 and 64.  path: 0
 * picks the kernel (a tuned one for B = 128, G = 64 at every index width,
 * the general one otherwise); 1 runs the general kernel for every layout
 * (the results are the same; for tests and measurement).  PA_ERR_ARG for
 * any other value or layout. */
typedef struct {
  int v_bits;
  double m_step_factor;
  unsigned long long seed;
  int block_size;
  int m_block_size;
  int path;
} pa_turbo_config;

/* Persistent bytes of one tensor's TurboAdam state at the default layout
 * (the page's ledger: for 131,072 values with both representations,
 * 36,876 + 69,632 = 106,508), and at any layout above.  0 for an index
 * width or layout the step does not take. */
size_t pa_turbo_state_bytes(int compress_m, int compress_v, int v_bits, size_t n);
size_t pa_turbo_layout_bytes(int compress_m, int compress_v, int v_bits, int block_size, int m_block_size,
                             size_t n);

/* Device workspace a pa_turbo_step_list call needs, for every tensor with
 * compress_m: one double per 256 values (its residual partial sums) plus
 * one per 2048 of those partial sums (their chunk sums).  The contents need
 * no initialisation and are dead after the call. */
size_t pa_turbo_workspace_bytes(size_t count, const pa_turbo_state* states, const size_t* n);

/* One TurboAdam step over `count` tensors sharing hyper, config and step
 * (1 to 2^32 - 1, counting this update; PA_ERR_ARG outside): one launch over
 * all tensors (the tuned kernel: a wavefront per 256 values; the general
 * one: a workgroup per 1024 values; both in dispatch order), then one
 * workgroup per 2048 residual partial sums and one per UState tensor that
 * completes the sum and rotates its scales.  `states` is a host array of count
 * descriptors; `workspace` a device buffer of at least
 * pa_turbo_workspace_bytes (8-byte aligned).  The launch plan is cached per
 * distinct list of parameter and state pointers, sizes and configuration
 * (see pa_release_plans), its gradient pointers written into it when they
 * move, as for pa_step_list.  Written buffers may not overlap each other,
 * the gradients or the workspace (PA_ERR_ALIAS).  hyper's non-finite
 * counter, gradient scale and skip flag work as for pa_step.  Once a
 * list's plan exists, a call enqueues its kernels and nothing else, so it
 * can be captured in a HIP graph (a captured call keeps its step, scalars
 * and gradients). */
int pa_turbo_step_list(size_t count, float* const* params, const float* const* grads, const pa_turbo_state* states,
                       const size_t* n, const pa_hyper* hyper, const pa_turbo_config* config, long long step,
                       void* workspace, size_t workspace_bytes, void* stream);

/* pa_turbo_step_list with 16-bit parameters and/or gradients (the TurboAdam
 * package page, Verification: its tests run fp16, bf16 and fp32
 * parameters).  The pairs of pa_step_typed: (F32, F32), (BF16, BF16),
 * (F16, F16), (BF16, F32), (F16, F32); PA_ERR_ARG for any other.  The
 * update runs in FP32 exactly as for FP32 tensors: 16-bit values widen
 * exactly and only the new parameter is rounded back to its type, to
 * nearest even, so the state (which never depends on the parameters) is
 * the state of the FP32 step on the widened values.  params[i] and
 * grads[i] hold n[i] elements of their type (bfloat16 / binary16 as uint16
 * bit patterns), aligned to four elements (16 bytes for FP32, 8 for 16-bit
 * types; PA_ERR_ALIGN otherwise).  All other arguments, results and errors
 * as for pa_turbo_step_list, which is the (F32, F32) case. */
int pa_turbo_step_list_typed(int param_dtype, int grad_dtype, size_t count, void* const* params,
                             const void* const* grads, const pa_turbo_state* states, const size_t* n,
                             const pa_hyper* hyper, const pa_turbo_config* config, long long step, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Persistent optimizer-state bytes for n parameters in `mode` (the state
 * ledger; Packed AdamW Reference README, "The narrow result": 8 bytes per
 * parameter for FP32 AdamW, 4 for the packed word).  Blockwise: two code
 * bytes per parameter plus two FP32 absmax values per 2048-block (n must be
 * a multiple of 2048).  Returns 0 for an unknown mode. */
size_t pa_state_bytes(int mode, size_t n);

/* Description of one mode's lanes (for inspection and tests): the Packed
 * AdamW Reference README, introduction (E4M11 signed first moment, E4M12
 * unsigned RMS, the FP16-first/FP16-RMS comparison word) and its section
 * "Dependency-light inspection"; the KBench reference's 2048-element blocks
 * of 8-bit codes.  Exponent bias 15 of the E4 lanes is this library's
 * reading (the pages do not print it).  PA_ERR_ARG for a null `out` or an
 * unknown mode. */
typedef struct {
  int mode;
  int lanes;              /* values per parameter in the persistent state */
  int m_sign_bits, m_exp_bits, m_mant_bits, m_exp_bias;
  int r_sign_bits, r_exp_bits, r_mant_bits, r_exp_bias;
  double m_max, m_min_normal, m_min_subnormal;
  double r_max, r_min_normal, r_min_subnormal;
  int block;              /* 2048 for PA_BLOCKWISE8, else 0 */
} pa_format;

int pa_format_info(int mode, pa_format* out);

/* Text for a status code (static storage). */
const char* pa_status_string(int status);

/* The hipError_t of the last failed HIP call made by the library in this
 * thread (0 if none). */
int pa_last_hip_error(void);

/* Free every cached launch-plan table and blockwise table buffer (device
 * memory).  Waits for the device first.  Safe to call at any time outside a
 * running call. */
void pa_release_plans(void);

/* Plan-cache self-test export (host only): the number of cached launch
 * plans of list steps, of gradient pre-passes and of TurboAdam steps.  A
 * plan is cached per list of parameters and state buffers (and lengths);
 * gradients that move between calls reuse it.  PA_ERR_ARG for a null
 * pointer. */
int pa_debug_plan_count(int* step_plans, int* stats_plans, int* turbo_plans);

/* Blockwise launch self-test export (host only, for the tests of both
 * launches): 0 (the default) chooses by size as pa_step_list describes; -1
 * takes the persistent launch at every size; k >= 1 takes the ordered launch
 * with k blocks per workgroup at every size (the persistent launch still
 * serves pa_step_list_noalloc and calls under graph capture).  Applies to
 * every later call in the process.  PA_ERR_ARG below -1 or above 2^20. */
int pa_debug_blockwise_path(long long blocks_per_workgroup);

/* Scalar self-test export (host only, no device work): the per-call
 * binary32 scalars the kernels receive, formed from `hyper` and `step`
 * exactly as every step entry point forms them (KBench quantized-optimizer-
 * state reference, `quantized_adamw_step`: the bias corrections and their
 * quotients are Python floats that meet the FP32 tensors).  out (host, 9
 * floats): beta1, 1-beta1, beta2, 1-beta2, 1-beta2^t, lr/(1-beta1^t),
 * 1-lr*wd and eps, each formed in double and rounded once to binary32, then
 * beta1 * 2^112 (exact: the factor that meets the E4 first moment decoded
 * without its 2^-112 scale); *inv_bc2 (host) = 1/(the binary32 1-beta2^t)
 * rounded to double (the quotient v'/bc2 is taken as a product with it).
 * Validates hyper and step as pa_step does (PA_ERR_ARG, PA_ERR_ALIGN);
 * null out or inv_bc2 is PA_ERR_ARG. */
int pa_debug_scalars(const pa_hyper* hyper, long long step, float* out, double* inv_bc2);

/* Codec self-test export: apply one lane codec of the GPU path to n device
 * values.  lane 0 = E4M11 first moment, 1 = E4M12 RMS, 2 = binary16,
 * 3 = bfloat16 (the 16-bit parameter and blockwise output rounding).
 * dir 0 encodes float -> uint16 (in: float*, out: uint16_t*), dir 1 decodes
 * uint16 -> float.  Device pointers, asynchronous on `stream`.  Used by the
 * tests to check every code of every lane on the device. */
int pa_debug_codec(int lane, int dir, const void* in, void* out, size_t n, void* stream);

/* Square-root self-test export: out[i] = the GPU path's correctly rounded
 * binary32 square root of in[i], for n device floats, asynchronous on
 * `stream`.  The update takes sqrt(v'/bc2) and sqrt(v') with this routine;
 * the tests compare it with the host's IEEE square root on every float. */
int pa_debug_sqrt(const float* in, float* out, size_t n, void* stream);

/* 1Q endpoint self-test export: for n positive finite device floats in[i],
 * out[i] = binary16 of log2(in[i]) rounded down (low 16 bits) and up (high
 * 16 bits), as the TurboAdam step computes a block's endpoints (TurboAdam
 * package page, 1Q).  The tests compare it with the oracle on every
 * positive binary32.  Asynchronous on `stream`. */
int pa_debug_q1_ends(const float* in, uint32_t* out, size_t n, void* stream);

/* 1Q level self-test export: for n device endpoint words ends[i] (low 16
 * bits the fp16 lower log2 endpoint, high 16 bits the upper one) and
 * L = 2^bits (bits 2, 3, 4, 6 or 8), out[i*L + k] = level k of that block as the
 * TurboAdam step decodes it (TurboAdam package page, 1Q): 0 for k = 0, else
 * the exact power 2^x, x = lo + (hi - lo)(k - 1)/(L - 2) in double, rounded
 * once to binary32.  exact = 0 takes the step's own table builders (the
 * device exp2, or for 8-bit indices a geometric recurrence, with a
 * double-double evaluation deciding near binary32 midpoints); exact != 0
 * takes every level through the double-double evaluation.  out
 * holds n*L floats.  PA_ERR_ARG for another width, null pointers or
 * n > 2^40.  Asynchronous on `stream`. */
int pa_debug_q1_levels(const uint32_t* ends, int bits, int exact, float* out, size_t n, void* stream);

/* 1Q level rounding self-test export: out[i] = RN32(2^x[i]), the exact
 * power of two of the double x[i] rounded once to binary32 (TurboAdam
 * package page, 1Q: the grid levels), for n device doubles.  exact = 0
 * takes the route of the 2- and 4-bit tables (the device exp2 decides when
 * every value within 2^-48 of its result rounds alike, else the
 * double-double evaluation); exact != 0 takes the double-double evaluation
 * alone.  x 8-byte aligned, out 4-byte aligned (PA_ERR_ALIGN), non-null
 * (PA_ERR_ARG).  Asynchronous on `stream`. */
int pa_debug_pow2_rn32(const double* x, int exact, float* out, size_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
