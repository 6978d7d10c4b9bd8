/*
 * qknr.h -- C ABI of the fused in-place QK RMSNorm + rotary position embedding
 * for AMD MI355X (gfx950).
 *
 * The operation is the one described by the page "SGLang Diffusion fused
 * operator fused_inplace_qknorm_rope: in-depth technical analysis"
 * (m.lsln.cn/news/241376):
 *   - section 2.1: per (token, head) vector x of length head_dim,
 *       n_i = x_i * rsqrt(sum_j x_j^2 / head_dim + eps) * w_i
 *     with w = q_weight for Q heads and k_weight for K heads;
 *   - section 2.2: the first rope_dim dims of n are rotated pairwise by the
 *     angles of cache row positions[token], laid out as
 *       [cos_0 .. cos_{R/2-1} | sin_0 .. sin_{R/2-1}]  (fp32, R = rope_dim),
 *     pairing (2j, 2j+1) when is_neox == 0 (interleaved, GPT-J) and
 *     (j, j + R/2) when is_neox != 0 (NeoX); a pair (a, b) becomes
 *     (a*cos_j - b*sin_j, b*cos_j + a*sin_j); dims >= rope_dim pass through;
 *   - section 2.3: all of it in one pass, fp32 arithmetic in registers,
 *     result rounded (to nearest even) to the I/O type and written in place;
 *   - section 3 (I/O contract): q [T, Hq, D] and k [T, Hkv, D] fp16/bf16 with
 *     innermost stride 1 (GQA: Hq != Hkv allowed), weights [D] of the same
 *     dtype, the cos|sin cache [rows, R] fp32 row-contiguous, positions [T]
 *     int32 or int64.
 *
 * Supported shapes: head_dim from 2 to 512 and rope_dim even with
 * 2 <= rope_dim <= head_dim, either pairing; qknr_can_use reports exactly this
 * set, a superset of the page's (section 4.6 compile-time guards, section 5.2
 * predicate: head_dim in {64, 128, 256}, rope_dim a multiple of head_dim/32,
 * for NeoX rope_dim/(head_dim/32) a power of two >= 2). Two kernels serve it:
 *   - the vectorised kernel (16-byte lanes, or half or a full wave per head,
 *     several heads per wave instruction), taken whenever all of these hold:
 *     head_dim a multiple of 8 in [16, 512]; for NeoX, rope_dim/2 a multiple
 *     of a lane width E (8 for any head_dim; also head_dim/32 and
 *     head_dim/64 >= 2 for head_dim 64, 128, 256), or, for the fused op and
 *     the LayerNorm sibling, any even rope_dim/2 (16-byte lanes whose partners
 *     sit 2, 4 or 6 slots over in a neighbouring lane when rope_dim/2 is not a
 *     multiple of 8; at head_dim 96 with rope_dim/2 a multiple of 6 but
 *     not of 8, 12-byte lanes, 16 per head, instead);
 *     q, k, weights (and biases) 16-byte aligned and every used q/k
 *     stride a multiple of 16 bytes; lane offsets inside a head group below
 *     2^31 bytes (a mapping with fewer heads per group is tried first); and,
 *     for the unfused steps, head_dim 64, 128 or 256;
 *   - the element-granular kernel for every other supported case, with
 *     2-, 4-, 8- or 16-byte accesses: 2*r bytes need head_dim a multiple of r
 *     and q, k, weights (and biases) and every used stride 2*r-byte aligned. A
 *     head takes L lanes of S runs of r elements (L*S*r >= head_dim, S*r <= 8)
 *     and a wave instruction 64/L heads; of the allowed (r, S, L) -- L a power
 *     of two, or the exact lane count a head needs -- it takes the one with
 *     the fewest wave instructions per token, then a power-of-two L, the
 *     wider access, fewer slots. Several heads per instruction need their
 *     lane offsets below 2^31 bytes; otherwise one head per instruction (no
 *     stride limit). It needs only element alignment and computes the same
 *     formulas.
 * qknr_inplace_ex reports which one a call takes (qknr_launch_info.generic).
 *
 * All entry points are thread-safe and keep no state besides small per-device
 * caches of the CU count and kernel occupancy.
 */
#ifndef QKNR_H
#define QKNR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKNR_API __attribute__((visibility("default")))

/* Status codes. Every rejection happens before any HIP call or enqueue, so a
 * rejected call leaves q and k untouched. */
enum {
  QKNR_OK = 0,
  QKNR_E_NULL = -1,        /* a required pointer is NULL */
  QKNR_E_SHAPE = -2,       /* negative size or stride, overlapping head views, size overflow */
  QKNR_E_UNSUPPORTED = -3, /* (head_dim, rope_dim) outside the supported set */
  QKNR_E_ALIGN = -4,       /* q/k/weights/biases or q/k strides not multiples of 2 bytes,
                              cache not 4-byte aligned, positions not aligned to their type */
  QKNR_E_DTYPE = -5,       /* unknown dtype or pos_dtype code */
  QKNR_E_ARG = -6,         /* eps negative or not finite; bad launch configuration */
  QKNR_E_LAUNCH = -7,      /* the HIP runtime refused the launch */
  QKNR_E_DEVICE = -8       /* querying the current device failed */
};

/* I/O element types of q, k and the weights. */
enum { QKNR_BF16 = 0, QKNR_FP16 = 1 };
/* Element types of positions. */
enum { QKNR_I32 = 0, QKNR_I64 = 1 };

/*
 * qknr_inplace -- apply the fused QK RMSNorm + RoPE to q and k in place.
 *
 *   q, k            device pointers to element [0,0,0] of q and k. Element
 *                   (t, h, i) of q lives at  q + t*q_tok_stride_B
 *                   + h*q_head_stride_B + 2*i  (bytes); likewise for k.
 *                   Strides are in BYTES, must be >= 0, even (multiples of 16
 *                   for the vectorised kernel) and describe non-overlapping
 *                   head vectors. Any layout works
 *                   (contiguous [T,H,D], strided views into a fused qkv buffer,
 *                   head-major); only the T*(Hq+Hkv)*head_dim Q/K elements are
 *                   read and written, no other byte.
 *   wq, wk          device pointers to the [head_dim] RMSNorm weights of Q and
 *                   of K, in the I/O dtype (16-byte aligned for the vectorised
 *                   kernel).
 *   cos_sin_cache   device pointer to the fp32 table, row p at
 *                   cos_sin_cache + p*rope_dim; it must hold every row that
 *                   positions[] names (not checked: an out-of-range position
 *                   is undefined behaviour, as in the source design).
 *   positions       device pointer to T positions, int32 or int64 (pos_dtype).
 *   T, Hq, Hkv      tokens, Q heads, K heads. T == 0 or Hq + Hkv == 0 is a
 *                   no-op returning QKNR_OK (pointers are not inspected).
 *   head_dim, rope_dim, is_neox   see "Supported shapes" above.
 *   eps             added to the mean square; finite and >= 0 (passed as fp32).
 *   dtype           QKNR_BF16 or QKNR_FP16 (q, k, wq, wk).
 *   pos_dtype       QKNR_I32 or QKNR_I64.
 *   stream          HIP stream of the current device; the work is enqueued
 *                   there and the call returns without waiting.
 *
 * Ownership: all buffers belong to the caller; the library allocates, frees
 * and retains nothing. q and k must not overlap each other (not checked).
 * Returns QKNR_OK once enqueued, or a negative status (see above).
 */
QKNR_API int32_t qknr_inplace(void* q, void* k, const void* wq, const void* wk,
                              const float* cos_sin_cache, const void* positions,
                              int64_t T, int32_t Hq, int32_t Hkv,
                              int32_t head_dim, int32_t rope_dim, int32_t is_neox,
                              float eps,
                              int64_t q_tok_stride_B, int64_t q_head_stride_B,
                              int64_t k_tok_stride_B, int64_t k_head_stride_B,
                              int32_t dtype, int32_t pos_dtype, hipStream_t stream);

/*
 * Launch configuration of qknr_inplace_ex. Zero in any field means "choose
 * automatically" (what qknr_inplace does; the automatic values are given in
 * brackets).
 *   lanes_per_head   lanes of the 64-lane wavefront that share one head vector:
 *                    head_dim/8 (16-byte accesses per lane), 32 (half a wave)
 *                    or 64 (a full wave; head_dim 128 and 256 only). NeoX needs
 *                    rope_dim/2 to be a multiple of head_dim/lanes_per_head.
 *                    [the first of head_dim/8, 32, 64 that fits the pairing and
 *                    the lane-offset limit; none: the element-granular kernel]
 *                    Other head_dims take only their automatic mapping (0, or
 *                    its lane count as qknr_launch_info reports it): head_dim/8
 *                    lanes padded to a power of two, or exact-fit groups of
 *                    head_dim/8 lanes, or 16 lanes of 12 bytes at head_dim 96.
 *   groups_per_item  head groups (one per wave instruction: 64/lanes_per_head
 *                    heads of one token) that a wave handles per work item;
 *                    a work item never spans two tokens. [2; 4 for "long
 *                    items": a head_dim other than 64/128/256 with NeoX
 *                    pairing, or whose head group holds at most 640 bytes.
 *                    Left automatic, the fused op on 16-byte lanes (not in
 *                    exact-fit groups) with at least 3 items per token ends
 *                    on ceil(2048 / n) tokens whose items hold half as many
 *                    groups (n such items per token), if the launch has at
 *                    least 8 times that many tokens; qknr_launch_info.items
 *                    counts them]
 *   unroll           head groups loaded before the first is computed: 1, 2 or 4.
 *                    [2; 4 for long items, except head_dim 40 in exact-fit
 *                    groups of 5 lanes with NeoX partners 4 slots over, which
 *                    keeps 2] A head_dim other than 64/128/256 runs at 2 or 4
 *                    (1 runs as 2).
 *   block_waves      wavefronts per workgroup: 1..8. [3 when a head takes at
 *                    most 16 lanes; 6 at head_dim 256 with 16-byte lanes
 *                    (32 lanes per head; the LayerNorm sibling keeps 4); 2
 *                    for long items; else 4, also on the element-granular
 *                    kernel]
 *   max_blocks       0: one workgroup per block_waves work items, each wave
 *                    handles one item [default; on the element-granular
 *                    kernel, instances that keep at most 6 waves per SIMD
 *                    resident take the persistent grid]; -1: a persistent grid
 *                    of (occupancy x CUs) workgroups striding over the items;
 *                    > 0: at most that many workgroups, striding.
 *   generic          1: take the element-granular kernel even where the
 *                    vectorised one applies (lanes_per_head must then be 0);
 *                    0: choose [0].
 * On the element-granular kernel a group is the 64/L heads of one wave
 * instruction (see "Supported shapes"): groups_per_item is the groups per work
 * item [twice the groups loaded together], block_waves and max_blocks apply as
 * above [4 waves], unroll is set by the kernel instance (16/(S*r) groups loaded
 * before the first is computed, with S slots of r elements per lane; reported
 * in qknr_launch_info.unroll; any valid value is accepted), and lanes_per_head
 * must be 0 (an explicit lane mapping that the case cannot use is
 * QKNR_E_ARG).
 */
typedef struct qknr_launch_cfg {
  int32_t lanes_per_head;
  int32_t groups_per_item;
  int32_t unroll;
  int32_t block_waves;
  int32_t max_blocks;
  int32_t generic;
} qknr_launch_cfg;

/* What a call launches (filled by qknr_inplace_ex, also for empty work, where
 * grid_blocks stays 0). On the element-granular kernel (generic = 1) a lane
 * owns elems_per_lane elements in runs of access_bytes/2 (1, 2, 4 or 8),
 * lanes_per_head lanes apart, and heads_per_wave heads share a wave
 * instruction. access_bytes was added in the struct's former tail padding: the
 * size (48 bytes) and the other offsets are unchanged. */
typedef struct qknr_launch_info {
  int32_t lanes_per_head;
  int32_t elems_per_lane;
  int32_t heads_per_wave;
  int32_t groups_per_token;
  int32_t groups_per_item;
  int32_t unroll;
  int32_t block_threads;
  int32_t grid_blocks;
  int64_t items;
  int32_t generic;
  int32_t access_bytes; /* bytes per Q/K load or store of a lane */
} qknr_launch_info;

/* qknr_inplace with an explicit launch configuration (cfg may be NULL) and an
 * optional report of what was launched (info may be NULL). Same contract and
 * status codes as qknr_inplace; an invalid cfg field returns QKNR_E_ARG. */
QKNR_API int32_t qknr_inplace_ex(void* q, void* k, const void* wq, const void* wk,
                                 const float* cos_sin_cache, const void* positions,
                                 int64_t T, int32_t Hq, int32_t Hkv,
                                 int32_t head_dim, int32_t rope_dim, int32_t is_neox,
                                 float eps,
                                 int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                 int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                 int32_t dtype, int32_t pos_dtype, hipStream_t stream,
                                 const qknr_launch_cfg* cfg, qknr_launch_info* info);

/*
 * The unfused chain that the fused op replaces (section 2.4: two launches, the
 * normalised values written to memory in the I/O type and read back; section 6:
 * the fallback path runs a QK RMSNorm and then a RoPE in place). These exist as
 * a measured baseline for the fused op; each step rounds its own output.
 *
 * qknr_rmsnorm_inplace -- section 2.1 only: q and k (same layout rules as
 *   qknr_inplace) are replaced by x * rsqrt(mean(x^2) + eps) * w, rounded to the
 *   I/O type. No cache, positions or rotation arguments; head_dim 2..512.
 * qknr_rope_inplace -- section 2.2 only: the first rope_dim dims of every head
 *   of q and k are rotated by cache row positions[t] as stored (no norm); no
 *   weights or eps.
 * qknr_unfused_inplace -- same arguments and result contract as qknr_inplace,
 *   computed as qknr_rmsnorm_inplace followed by qknr_rope_inplace on the same
 *   stream (two launches, the intermediate rounded to the I/O type). Every
 *   argument is validated before either launch; if the second launch is refused
 *   (QKNR_E_LAUNCH), q and k hold the normalised, unrotated values.
 * Status codes and ownership as for qknr_inplace.
 */
QKNR_API int32_t qknr_rmsnorm_inplace(void* q, void* k, const void* wq, const void* wk,
                                      int64_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                      float eps,
                                      int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                      int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                      int32_t dtype, hipStream_t stream);
QKNR_API int32_t qknr_rope_inplace(void* q, void* k, const float* cos_sin_cache,
                                   const void* positions, int64_t T, int32_t Hq, int32_t Hkv,
                                   int32_t head_dim, int32_t rope_dim, int32_t is_neox,
                                   int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                   int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                   int32_t dtype, int32_t pos_dtype, hipStream_t stream);
QKNR_API int32_t qknr_unfused_inplace(void* q, void* k, const void* wq, const void* wk,
                                      const float* cos_sin_cache, const void* positions,
                                      int64_t T, int32_t Hq, int32_t Hkv,
                                      int32_t head_dim, int32_t rope_dim, int32_t is_neox,
                                      float eps,
                                      int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                      int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                      int32_t dtype, int32_t pos_dtype, hipStream_t stream);

/*
 * qknr_layernorm_rope_inplace -- the per-head QK LayerNorm sibling (the SGLang
 * "Kernel Design Agent (KDA)" kernel-directory article, FLUX.2 fused producers:
 * a per-head LayerNorm of Q and K): every head vector x of q and k becomes
 *   (x - mean(x)) * rsqrt(mean((x - mean(x))^2) + eps) * w + b
 * (biased variance, fp32 arithmetic, one rounding to the I/O type), followed,
 * when rope_dim > 0, by the same rotation as qknr_inplace. rope_dim == 0 means
 * the norm alone (cos_sin_cache, positions, is_neox and pos_dtype are then
 * ignored and may be NULL/0). bq, bk: the [head_dim] bias rows of Q and K in
 * the I/O dtype, or both NULL for no bias. Same layout rules,
 * supported shapes, status codes and ownership as qknr_inplace (with
 * rope_dim == 0, any head_dim from 2 to 512).
 */
QKNR_API int32_t qknr_layernorm_rope_inplace(void* q, void* k, const void* wq, const void* wk,
                                             const void* bq, const void* bk,
                                             const float* cos_sin_cache, const void* positions,
                                             int64_t T, int32_t Hq, int32_t Hkv,
                                             int32_t head_dim, int32_t rope_dim, int32_t is_neox,
                                             float eps,
                                             int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                             int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                             int32_t dtype, int32_t pos_dtype, hipStream_t stream);

/* qknr_layernorm_rope_inplace with an explicit launch configuration (cfg may
 * be NULL) and an optional report of what was launched (info may be NULL),
 * as qknr_inplace_ex is to qknr_inplace. The LayerNorm instances at head_dim
 * 64, 128 and 256 exist at unroll 2 only (another unroll value runs as 2);
 * the fields mean what they mean for qknr_inplace_ex. Same contract and
 * status codes as qknr_layernorm_rope_inplace. */
QKNR_API int32_t qknr_layernorm_rope_inplace_ex(void* q, void* k, const void* wq, const void* wk,
                                                const void* bq, const void* bk,
                                                const float* cos_sin_cache, const void* positions,
                                                int64_t T, int32_t Hq, int32_t Hkv,
                                                int32_t head_dim, int32_t rope_dim,
                                                int32_t is_neox, float eps,
                                                int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                                int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                                int32_t dtype, int32_t pos_dtype,
                                                hipStream_t stream, const qknr_launch_cfg* cfg,
                                                qknr_launch_info* info);

/*
 * qknr_can_use -- 1 if qknr_inplace supports this combination, else 0: the
 * "Supported shapes" set above (a superset of the page's capability predicate,
 * section 5.2), with known dtype and pos_dtype codes. Pure host function, no
 * HIP call.
 */
QKNR_API int32_t qknr_can_use(int32_t head_dim, int32_t rope_dim, int32_t is_neox,
                              int32_t dtype, int32_t pos_dtype);

/* Static, never-freed description of a status code ("unknown status" for
 * codes not listed above). Pure host function. The Python binding raises an
 * exception carrying this text whenever a call returns a non-zero status: the
 * SGLang Kernel Design Agent (KDA) kernel-directory page, in its maintenance
 * rules ("directory maintenance conventions and extension guide", rule 3),
 * asks that a public kernel come with a can_use predicate and fail by raising
 * rather than by returning None, which callers forget to check. */
QKNR_API const char* qknr_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* QKNR_H */
