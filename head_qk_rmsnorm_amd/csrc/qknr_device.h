// qknr_device.h -- device code of the fused in-place QK RMSNorm + rotary
// position embedding for MI355X (gfx950), shared by the kernel-instantiation
// sources (qknr_inst.hip, built once per I/O type and instance group) and the
// host library (qknr.hip).
//
// The operation follows the page "SGLang Diffusion fused operator
// fused_inplace_qknorm_rope: in-depth technical analysis" (m.lsln.cn/news/241376):
// section 2.1 (per-head RMSNorm with a learned weight), section 2.2 (cos|sin
// cache rows, interleaved and NeoX pairing, partial rotary), section 2.3 (the
// fused per-head flow: load, widen to fp32, sum of squares, rsqrt, scale,
// rotate, narrow, store in place) and section 3 (tensor contract). The C ABI is
// declared in include/qknr.h.
//
// Design for the 64-lane CDNA4 wavefront (the page's kernel is a 32-lane
// warp-per-head CUDA design; only its arithmetic is kept):
//   * L = head_dim / E lanes share one head vector, each lane owning E
//     contiguous elements. E = 8 gives 16-byte accesses per lane (L = 8, 16, 32
//     for head_dim 64, 128, 256: 8, 4 or 2 heads per wave instruction). Half a
//     wave (L = 32) and a full wave (L = 64) per head are the other mappings;
//     half a wave also covers the NeoX rotary widths whose rotary lanes would
//     not be a power of two with E = 8.
//   * A wave's work item is a run of head groups of ONE token, so the position
//     is wave-uniform and read with a scalar load; each lane loads the cos/sin
//     values of its own dims once per item and keeps them in registers for
//     every head of the item.
//   * The fp32 sum of squares is reduced over the L lanes of a head with DPP
//     row operations (quad_perm, row_half_mirror, row_mirror), one ds_swizzle
//     across 16-lane rows for L >= 32 and two readlanes across the wave halves
//     for L = 64; every lane of a head ends with the bit-identical sum.
//   * NeoX partners sit m = (rope_dim/2)/E lanes up or down within the same
//     head; they are fetched with ds_bpermute.
//   * A wave instruction covers one head group: heads of Q or of K (never
//     both) of one token, so the group's base address is wave-uniform (an SGPR
//     buffer descriptor) and each lane adds a fixed 32-bit offset. Only Q/K
//     elements are loaded or stored.
//   * A wave's first memory requests are the loads of `unroll` head groups;
//     the weight rows, the position and the position-dependent cos/sin fetch
//     follow, so the head data is in flight while that chain resolves (issuing
//     the weights and the position first made every wave wait for them before
//     its head loads: 0.5-2.6% slower). Q/K traffic is streamed with
//     nontemporal loads and stores (each byte is touched once).
//   * By default every wave takes one work item and exits (no persistent grid):
//     the dispatcher back-fills CUs as waves finish, which balances the tail.
// Nothing here is a contraction, so there is no MFMA.

#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qknr.h"

namespace qknr_impl {

constexpr int kWave = 64;
constexpr int kMaxBlockWaves = 8;

// ==== fused-kernel device code begin (the measured kernel; its hash keys the
// ==== committed hardware-counter summaries)
// ----------------------------------------------------------------------------
// I/O element formats: two 16-bit values per dword, lower address in the low
// half. Widening is exact; narrowing rounds to nearest even (gfx950
// v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
// ----------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct Bf16 {
  static __device__ __forceinline__ void unpack(uint32_t u, float& lo, float& hi) {
    lo = __uint_as_float(u << 16);
    hi = __uint_as_float(u & 0xffff0000u);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

struct Fp16 {
  static __device__ __forceinline__ void unpack(uint32_t u, float& lo, float& hi) {
    f16x2_t v = __builtin_bit_cast(f16x2_t, u);
    lo = (float)v.x;
    hi = (float)v.y;
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// NV packed dwords (2*NV elements) owned by one lane.
template <int NV>
struct Raw {
  uint32_t w[NV];
};

template <int NV>
__device__ __forceinline__ Raw<NV> load_raw(const char* p) {
  Raw<NV> r;
  if constexpr (NV == 4) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (NV == 3) {
    const uint32_t* const d = reinterpret_cast<const uint32_t*>(p);
    r.w[0] = d[0]; r.w[1] = d[1]; r.w[2] = d[2];
  } else if constexpr (NV == 2) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    static_assert(NV == 1, "1, 2, 3 or 4 dwords per lane");
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  return r;
}

// ----------------------------------------------------------------------------
// Cross-lane helpers
// ----------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kSwizzleXor16 = 0x401F;  // ds_swizzle bit mode: and 0x1f, xor 0x10

// Sum over the L consecutive lanes of each head, for any L up to 32 with heads
// packed from lane 0 (exact-fit lane groups): a tree of partial sums toward
// the head's first lane, then a broadcast from it, so every lane of a head
// gets the same bits. Lanes past the last head compute unused values.
__device__ __forceinline__ float seg_sum(float v, int lane, int li, int L) {
  for (int s = 1; s < L; s <<= 1) {
    const float o = __int_as_float(
        __builtin_amdgcn_ds_bpermute(((lane + s) & 63) << 2, __float_as_int(v)));
    v += (li + s < L) ? o : 0.0f;
  }
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane - li) << 2, __float_as_int(v)));
}

// Sum over aligned groups of L lanes; every lane of a group gets the same bits.
// After the two quad steps a quad is uniform, so a mirror inside 8 (16) lanes
// adds exactly the other quad (half row).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L == 2 || L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "lanes per head");
  v += dpp_mov<kDppQuadXor1>(v);
  if constexpr (L >= 4) v += dpp_mov<kDppQuadXor2>(v);
  if constexpr (L >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (L >= 16) v += dpp_mov<kDppRowMirror>(v);
  if constexpr (L >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
  if constexpr (L == 64) {
    // both halves are uniform now; add them in the same order on every lane
    v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  }
  return v;
}

__device__ __forceinline__ float lane_fetch(int byte_addr, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(byte_addr, __float_as_int(v)));
}

// Order this wave's LDS accesses around a row exchange (a wave's LDS accesses
// execute in order; the fences keep the compiler from moving them).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// ----------------------------------------------------------------------------
// Kernel
// ----------------------------------------------------------------------------
// Q/K are read and written exactly once: nontemporal accesses keep them from
// displacing the reused weights, positions and cos|sin rows in L2. Stores also
// carry agent scope (sc1): they are written through to memory instead of
// staying dirty in the XCD's L2 until the end-of-kernel write-back, which
// shortens the drain of every launch (measured 0.4-2% faster across sizes).
// Q/K accesses go through raw buffer instructions: a wave-uniform descriptor
// (base address of the head group, in SGPRs) plus a 32-bit per-lane offset.
// Offsets stay below 2^31 (checked on the host), far inside the descriptor's
// range, so no access is out of range.
constexpr int kBufferFlags = 0x00020000;  // gfx9 raw-buffer descriptor word 3
constexpr int kCachePolicyNT = 2;          // cache-policy operand: nt
constexpr int kCachePolicySC1 = 16;        // cache-policy operand: sc1 (agent scope)
constexpr int kLoadPolicy = kCachePolicyNT;
constexpr int kStorePolicy = kCachePolicyNT | kCachePolicySC1;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, kBufferFlags);
}

template <int NV>
__device__ __forceinline__ Raw<NV> load_io(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  Raw<NV> r;
  if constexpr (NV == 4) {
    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kLoadPolicy));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (NV == 3) {
    const u32x3_t v = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, kLoadPolicy));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z;
  } else if constexpr (NV == 2) {
    const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kLoadPolicy));
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kLoadPolicy);
  }
  return r;
}

template <int NV>
__device__ __forceinline__ void store_io(__amdgpu_buffer_rsrc_t rs, uint32_t off, const Raw<NV>& r) {
  if constexpr (NV == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{r.w[0], r.w[1], r.w[2], r.w[3]}, rs, off, 0, kStorePolicy);
  } else if constexpr (NV == 3) {
    __builtin_amdgcn_raw_buffer_store_b96(u32x3_t{r.w[0], r.w[1], r.w[2]}, rs, off, 0, kStorePolicy);
  } else if constexpr (NV == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{r.w[0], r.w[1]}, rs, off, 0, kStorePolicy);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(r.w[0], rs, off, 0, kStorePolicy);
  }
}

typedef __attribute__((address_space(4))) const int32_t* cpos32_t;
typedef __attribute__((address_space(4))) const int64_t* cpos64_t;

__device__ __forceinline__ int64_t token_position(const void* pos, int pos64, int t) {
  return pos64 ? ((cpos64_t)pos)[t] : static_cast<int64_t>(((cpos32_t)pos)[t]);
}

struct Params {
  int64_t q_tok, k_tok;          // token strides (bytes)
  int64_t q_grp, k_grp;          // bytes between consecutive head groups (G head strides)
  uint32_t q_head, k_head;       // head strides (bytes); (G-1)*stride + 2*D fits 32 bits
  int32_t Hq, Hkv, R;
  int32_t D;                     // head_dim (instances with a run-time head_dim)
  float inv_d;                   // 1 / head_dim
  int32_t ngq;                   // Q head groups per token; K groups follow them
  int32_t pos64;
  int32_t cs_vec;                // cache rows 16-byte aligned and R/2 % 4 == 0
  int32_t has_bias;              // LayerNorm sibling: bias rows given
  float eps;
  int32_t ng, gpi, nc, n_items;  // groups per token, groups per item, items per token, items
  // Exact-fit lane groups (SEG instances): lanes per head, heads per wave
  // instruction. Instances that can end on shorter items (kTail): the first
  // such item (n_items: none) and its token; those items hold half the groups
  // of the others. (One pair of fields for both keeps the argument block at
  // its size: 16 more bytes cost the exact-fit instances 1-1.4%, though their
  // code was unchanged.)
  int32_t aux0, aux1;
};

// What a launch computes: the fused op, one of the two steps of the unfused
// chain it replaces (norm only: rotation skipped; rope only: the stored values
// are rotated as they are, no norm), or the per-head LayerNorm sibling with or
// without the rotation.
enum : int { kFused = 0, kNormOnly = 1, kRopeOnly = 2, kLayerRope = 3, kLayerOnly = 4 };

// One wave instruction covers one head group: G consecutive heads of Q, or of
// K, of one token (groups never mix Q and K), so the group's base address is
// wave-uniform and each lane adds a fixed 32-bit offset.
//
// DMAX is the head_dim the instance is built for. EXACT instances have
// head_dim == DMAX; the others take any multiple of E up to DMAX at run time
// (each head keeps a lane group of DMAX/E lanes, the spare ones masked).
// SHIFT 2, 4 or 6 (NeoX, 8 elements per lane): rope_dim/2 is that much more than
// a multiple of 8, so a partner sits SHIFT slots over in a neighbouring lane.
template <class IO, int DMAX, int E, bool NEOX, bool FULL, int U, int MODE, bool EXACT,
          int SHIFT = 0, bool SEG = false>
__global__ void __launch_bounds__(kMaxBlockWaves * kWave)
qknr_kernel(char* __restrict__ qb, char* __restrict__ kb, const void* __restrict__ wqp,
            const void* __restrict__ wkp, const float* __restrict__ cache,
            const void* __restrict__ posp, const void* __restrict__ bqp,
            const void* __restrict__ bkp, const Params p) {
  constexpr int LC = DMAX / E;    // lanes per head (lane group)
  constexpr int GC = kWave / LC;  // heads per wave instruction
  constexpr int NV = E / 2;     // packed dwords per lane
  constexpr int NCS = NEOX ? E : E / 2;  // cos (and sin) values per lane
  static_assert(DMAX % E == 0 && E % 2 == 0 && GC >= 1, "lane mapping");
  static_assert(!SEG || (!EXACT && E == 8), "exact-fit lane groups: run-time head_dims");
  static_assert(SHIFT == 0 || ((SHIFT == 2 || SHIFT == 4 || SHIFT == 6) && NEOX && E == 8),
                "partner slot shift");
  constexpr bool kShift26 = SHIFT == 2 || SHIFT == 6;
  constexpr bool kLayerMode = MODE == kLayerRope || MODE == kLayerOnly;
  // Shifted partners read the token's cos|sin row from a copy in LDS instead
  // of per-lane global loads (A/B: partners 2 or 6 slots over +5 to +16%,
  // 4 slots over +7 to +13%), except where the copy measured slower: the
  // LayerNorm sibling's exact-fit groups with partners 2 or 6 slots over
  // (head_dim 80 / rope_dim 20: -4.4%) and partners 4 slots over in lane
  // groups padded to 32 or 64 lanes (head_dim 136: -3.5%, LayerNorm -5.8%)
  // NeoX instances at head_dim 64 and 128 (16-byte lanes) of the fused op and
  // the LayerNorm sibling stage the row too (one coalesced copy per wave
  // instead of 4 vector loads per lane; A/B: GQA +1.2%, Partial +0.7%,
  // head_dim 64/128 NeoX +1.8/+1.9%; LayerNorm GQA +1.7%, Partial +3.2%);
  // interleaved DiT was level and head_dim 256 lost (Large -9%, 256
  // interleaved -7.6%), so they keep per-lane loads.
  constexpr bool kStageCs0 = SHIFT == 0 && (MODE == kFused || MODE == kLayerRope) && EXACT && E == 8 && NEOX && DMAX <= 128;
  constexpr bool kStageCs = kStageCs0 || (SHIFT == 4 && (EXACT || DMAX < 256)) || (kShift26 && !(kLayerMode && SEG));
  // per wave: with shifted partners the exchange row (kWave * E floats; SHIFT
  // 2/6) and then room for the token's cos|sin row (kCsRow floats); without
  // them (kStageCs0) the row alone (DMAX floats)
  extern __shared__ float shift_rows[];
  constexpr int kCsRow = SHIFT != 0 ? 512 : DMAX;
  constexpr int kXRow = SHIFT != 0 ? kWave * E : 0;
  constexpr int kShiftRow = kXRow + kCsRow;
  const int lane = threadIdx.x & (kWave - 1);
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  // SEG: exact-fit lane groups of head_dim/E lanes (p.aux0, any count up to
  // 32), p.aux1 heads per wave instruction, the lanes past them idle
  const int L = SEG ? p.aux0 : LC;
  const int G = SEG ? p.aux1 : GC;
  const int sub = SEG ? lane / L : lane / LC;  // head slot in the group
  const int li = lane - sub * L;               // lane inside the head
  const int d0 = li * E;     // first dim owned by this lane
  const int D = EXACT ? DMAX : p.D;
  const bool in_head = SEG ? sub < G : (EXACT || d0 < D);  // spare lanes
  const int R = FULL ? D : p.R;
  const int half = R / 2;
  const uint32_t q_off = static_cast<uint32_t>(sub) * p.q_head + d0 * 2;
  const uint32_t k_off = static_cast<uint32_t>(sub) * p.k_head + d0 * 2;

  constexpr bool kRotate = MODE == kFused || MODE == kRopeOnly || MODE == kLayerRope;
  constexpr bool kRms = MODE == kFused || MODE == kNormOnly;
  // launches of the fused op on 16-byte lanes with aligned partners may end
  // on items of half as many groups, from item p.aux0 (token p.aux1) on; the
  // other instances have none
  constexpr bool kTail = MODE == kFused && E == 8 && !SEG && SHIFT == 0;
  constexpr bool kLayer = MODE == kLayerRope || MODE == kLayerOnly;

  // Weights (and LayerNorm biases) of this lane's dims, kept packed; loaded
  // once, after the first head loads are in flight. The LayerNorm modes keep
  // the other order (weights, biases and the position requested first, the
  // position prefetched one item ahead): for them the late order costs
  // registers, a wave per SIMD, and measured 1-3.5% slower on the NeoX
  // workloads.
  Raw<NV> wq_p{}, wk_p{}, bq_p{}, bk_p{};
  bool have_w = false;
  auto load_weights = [&]() {
    if constexpr (kRms || kLayer) {
      if (in_head) {
        wq_p = load_raw<NV>(static_cast<const char*>(wqp) + d0 * 2);
        wk_p = load_raw<NV>(static_cast<const char*>(wkp) + d0 * 2);
      }
    }
    if constexpr (kLayer) {
      if (in_head && p.has_bias) {
        bq_p = load_raw<NV>(static_cast<const char*>(bqp) + d0 * 2);
        bk_p = load_raw<NV>(static_cast<const char*>(bkp) + d0 * 2);
      }
    }
  };
  if constexpr (kLayer) {
    load_weights();
    have_w = true;
  }

  // NeoX: this lane holds dims d0..d0+E-1. With m = (R/2)/E, lanes below m
  // hold first-half dims and find their partners d + R/2 at the same offsets
  // in lane + m; lanes m..2m-1 hold the second half and look m lanes down.
  // Lanes from 2m on hold pass-through dims. Lower-half lanes subtract.
  // With rope_dim == head_dim every lane rotates: the spare lanes of a
  // run-time head_dim compute values that are never stored, and read cos/sin
  // column 0 so they stay inside the row.
  int partner_addr = lane << 2, j0 = 0;
  bool lower = false, lane_rot = true;
  if constexpr (NEOX && SHIFT == 0) {
    const int m = half / E;
    lane_rot = FULL || li < 2 * m;
    lower = li < m;
    if (lane_rot) {
      partner_addr = (lower ? lane + m : lane - m) << 2;
      j0 = !in_head ? 0 : (lower ? d0 : d0 - half);
    }
  } else {
    j0 = in_head ? d0 / 2 : 0;
  }
  // SHIFT 4, with R/2 = 8m + 4: slots 0-3 and 4-7 of a lane are runs of 4
  // dims that each lie in one half (R/2 is a multiple of 4), and the rotated
  // dims end on a lane boundary (R = 16m + 8). A first-half run k pairs with
  // slots (i+4)&7 of lane li+m+k, a second-half run with lane li-m-1+k, so
  // partner lane, cos/sin column and sign are kept per run. Lanes that do not
  // rotate (pass-through dims, spare lanes) fetch from themselves and read
  // columns 0-3, which keeps every access inside the head and the row.
  int pa_s[2] = {lane << 2, lane << 2}, jc_s[2] = {0, 0};
  bool lo_s[2] = {false, false}, ro_s = false;
  if constexpr (SHIFT == 4) {
    const int m = half >> 3;
    const int head_lane0 = lane - li;
    ro_s = in_head && d0 < 2 * half;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int d = d0 + 4 * k;
      const bool lo = d < half;
      const int pl = lo ? li + m + k : li - m - 1 + k;
      pa_s[k] = (ro_s ? head_lane0 + pl : lane) << 2;
      jc_s[k] = ro_s ? (lo ? d : d - half) : 0;
      lo_s[k] = lo;
    }
  }
  // SHIFT 2 or 6, with R/2 = 8m + SHIFT: a partner sits 2 or 6 slots over, and
  // the first and second halves of a lane would need different source
  // registers, so the normalised values go through this wave's row of LDS
  // instead (E floats per lane, lane-major: a head's dims are contiguous from
  // its first lane's slot). Pair (2p, 2p+1) of this lane reads the pair at its
  // partner dims, 8-byte aligned: R/2 and R are even, so a pair lies in one
  // half and on one side of the rotation end. Pairs that do not rotate (pass-
  // through dims, spare lanes) read themselves; cos/sin come as aligned pairs.
  int pidx[kShift26 ? E / 2 : 1];
  if constexpr (kShift26) {
    const int head0 = (lane - li) * E;
#pragma unroll
    for (int q2 = 0; q2 < E / 2; ++q2) {
      const int d = d0 + 2 * q2;
      const bool rot = in_head && d < 2 * half;
      pidx[q2] = rot ? head0 + (d < half ? d + half : d - half) : lane * E + 2 * q2;
    }
  }
  const bool ro_26[2] = {in_head && d0 < 2 * half, in_head && d0 + 4 < 2 * half};
  const bool cs_pairs = (reinterpret_cast<uintptr_t>(cache) & 7) == 0;

  auto head_sum = [&](float v) {
    if constexpr (SEG) {
      return seg_sum(v, lane, li, L);
    } else {
      return group_sum<LC>(v);
    }
  };

  const int total_waves = gridDim.x * wpb;
  int item = blockIdx.x * wpb + wib;
  if (item >= p.n_items) return;
  int64_t pos_next = 0;
  if constexpr (kLayer && kRotate) pos_next = token_position(posp, p.pos64, item / p.nc);

  for (; item < p.n_items; item += total_waves) {
    int t, g_begin, g_end;
    if (kTail && item >= p.aux0) {
      // the last items: half the groups each (the host ends launches on them
      // only with 2 or 4 groups per item), so the final waves are short
      const int half_gpi = p.gpi == 4 ? 2 : 1;
      const int tail_nc = p.gpi == 4 ? (p.ng + 1) >> 1 : p.ng;
      const int it = item - p.aux0;
      const int tt = it / tail_nc;
      t = p.aux1 + tt;
      g_begin = (it - tt * tail_nc) * half_gpi;
      g_end = min(g_begin + half_gpi, p.ng);
    } else {
      t = item / p.nc;
      g_begin = (item - t * p.nc) * p.gpi;
      g_end = min(g_begin + p.gpi, p.ng);
    }
    int64_t pos = 0;
    if constexpr (kLayer && kRotate) {
      pos = pos_next;
      if (item + total_waves < p.n_items)
        pos_next = token_position(posp, p.pos64, (item + total_waves) / p.nc);
    }
    char* const qrow = qb + t * p.q_tok;
    char* const krow = kb + t * p.k_tok;

    Raw<NV> raw[U];
    __amdgpu_buffer_rsrc_t rs[U];
    uint32_t off[U];
    bool ok[U], isk[U];
    auto issue = [&](int g) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int gu = g + u;
        isk[u] = gu >= p.ngq;  // wave-uniform
        const int gg = isk[u] ? gu - p.ngq : gu;
        rs[u] = head_rsrc(isk[u] ? krow + gg * p.k_grp : qrow + gg * p.q_grp);
        off[u] = isk[u] ? k_off : q_off;
        ok[u] = in_head && gu < g_end && gg * G + sub < (isk[u] ? p.Hkv : p.Hq);
        if (ok[u]) {
          raw[u] = load_io<NV>(rs[u], off[u]);
        } else {
#pragma unroll
          for (int w = 0; w < NV; ++w) raw[u].w[w] = 0u;
        }
      }
    };
    issue(g_begin);
    if constexpr (!kLayer) {
      // Nothing above waits on memory: the head loads leave before the weight
      // rows and the position (whose cos/sin fetch depends on it) are
      // requested, and the barrier keeps the scheduler from hoisting those
      // loads (and the waits they bring) above them.
      __builtin_amdgcn_sched_barrier(0);
      if (!have_w) {
        load_weights();
        have_w = true;
      }
      if constexpr (kRotate) pos = token_position(posp, p.pos64, t);
    }

    // cos / sin of this lane's dims at this token (loaded after the head data
    // is in flight; kept in registers for every group of the item)
    float cs[NCS], sn[NCS];
    if constexpr (kRotate) {
      const float* row = cache + pos * R;
      // the wave copies the row into LDS with coalesced loads (8-byte ones when
      // the table is 8-byte aligned; R is even), then each lane reads its own
      // columns from there
      // (an LDS pointer of its own: kept apart from the global row pointer so
      // that reads through it stay LDS instructions)
      float* const csr = shift_rows + wib * kShiftRow + kXRow;
      if constexpr (kStageCs) {
        wave_lds_fence();  // the previous item's reads of the row are done
        if (cs_pairs) {
          for (int c = 2 * lane; c < R; c += 2 * kWave)
            *reinterpret_cast<float2*>(csr + c) = *reinterpret_cast<const float2*>(row + c);
        } else {
          for (int c = lane; c < R; c += kWave) csr[c] = row[c];
        }
        wave_lds_fence();
      }
      if constexpr (kShift26) {
        // aligned pairs of this lane's columns (a pair never straddles a half)
#pragma unroll
        for (int q2 = 0; q2 < E / 2; ++q2) {
          const int d = d0 + 2 * q2;
          const bool lo = d < half;
          const int j = (in_head && d < 2 * half) ? (lo ? d : d - half) : 0;
          float c0, c1, s0, s1;
          if constexpr (kStageCs) {
            const float2 c2 = *reinterpret_cast<const float2*>(csr + j);
            const float2 s2 = *reinterpret_cast<const float2*>(csr + half + j);
            c0 = c2.x; c1 = c2.y; s0 = s2.x; s1 = s2.y;
          } else if (cs_pairs) {
            const float2 c2 = *reinterpret_cast<const float2*>(row + j);
            const float2 s2 = *reinterpret_cast<const float2*>(row + half + j);
            c0 = c2.x; c1 = c2.y; s0 = s2.x; s1 = s2.y;
          } else {
            c0 = row[j]; c1 = row[j + 1]; s0 = row[half + j]; s1 = row[half + j + 1];
          }
          cs[2 * q2] = c0; cs[2 * q2 + 1] = c1;
          sn[2 * q2] = lo ? -s0 : s0; sn[2 * q2 + 1] = lo ? -s1 : s1;
        }
      } else if constexpr (SHIFT == 4) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          if constexpr (kStageCs) {
            // columns jc and half + jc are multiples of 4: aligned 16-byte reads
            const float4 c4 = *reinterpret_cast<const float4*>(csr + jc_s[k]);
            const float4 s4 = *reinterpret_cast<const float4*>(csr + half + jc_s[k]);
            cs[4 * k] = c4.x; cs[4 * k + 1] = c4.y; cs[4 * k + 2] = c4.z; cs[4 * k + 3] = c4.w;
            sn[4 * k] = s4.x; sn[4 * k + 1] = s4.y; sn[4 * k + 2] = s4.z; sn[4 * k + 3] = s4.w;
          } else if (p.cs_vec) {
            const float4 c4 = *reinterpret_cast<const float4*>(row + jc_s[k]);
            const float4 s4 = *reinterpret_cast<const float4*>(row + half + jc_s[k]);
            cs[4 * k] = c4.x; cs[4 * k + 1] = c4.y; cs[4 * k + 2] = c4.z; cs[4 * k + 3] = c4.w;
            sn[4 * k] = s4.x; sn[4 * k + 1] = s4.y; sn[4 * k + 2] = s4.z; sn[4 * k + 3] = s4.w;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              cs[4 * k + i] = row[jc_s[k] + i];
              sn[4 * k + i] = row[half + jc_s[k] + i];
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sn[4 * k + i] = lo_s[k] ? -sn[4 * k + i] : sn[4 * k + i];
        }
      } else if (kStageCs0 && NCS % 4 == 0 && p.cs_vec) {
        const int jv = (FULL || NEOX || j0 < half) ? j0 : 0;
#pragma unroll
        for (int i = 0; i < NCS; i += 4) {
          const float4 c4 = *reinterpret_cast<const float4*>(csr + jv + i);
          const float4 s4 = *reinterpret_cast<const float4*>(csr + half + jv + i);
          cs[i] = c4.x; cs[i + 1] = c4.y; cs[i + 2] = c4.z; cs[i + 3] = c4.w;
          sn[i] = s4.x; sn[i + 1] = s4.y; sn[i + 2] = s4.z; sn[i + 3] = s4.w;
        }
      } else if (kStageCs0) {
#pragma unroll
        for (int i = 0; i < NCS; ++i) {
          const int j = (FULL || NEOX) ? j0 + i : min(j0 + i, half - 1);
          cs[i] = csr[j];
          sn[i] = csr[half + j];
        }
      } else if (NCS % 4 == 0 && p.cs_vec) {
        // interleaved with a partial rotation: R/2 is a multiple of 4 here, so a
        // lane's runs of 4 pairs are rotated whole or not at all; lanes past the
        // rotation read columns 0-3 (unused), which keeps the access in the row
        const int jv = (FULL || NEOX || j0 < half) ? j0 : 0;
#pragma unroll
        for (int i = 0; i < NCS; i += 4) {
          const float4 c4 = *reinterpret_cast<const float4*>(row + jv + i);
          const float4 s4 = *reinterpret_cast<const float4*>(row + half + jv + i);
          cs[i] = c4.x; cs[i + 1] = c4.y; cs[i + 2] = c4.z; cs[i + 3] = c4.w;
          sn[i] = s4.x; sn[i + 1] = s4.y; sn[i + 2] = s4.z; sn[i + 3] = s4.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCS; ++i) {
          const int j = (FULL || NEOX) ? j0 + i : min(j0 + i, half - 1);
          cs[i] = row[j];
          sn[i] = row[half + j];
        }
      }
      if constexpr (NEOX && SHIFT == 0) {
#pragma unroll
        for (int i = 0; i < NCS; ++i) sn[i] = lower ? -sn[i] : sn[i];
      }
    }

    for (int g = g_begin; g < g_end; g += U) {
      if (g != g_begin) issue(g);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[E];
#pragma unroll
        for (int w = 0; w < NV; ++w) IO::unpack(raw[u].w[w], x[2 * w], x[2 * w + 1]);
        float n[E];
        if constexpr (kLayer) {
          // two passes in registers: mean, then the variance of the centred values
          float sm = 0.0f;
#pragma unroll
          for (int i = 0; i < E; ++i) sm += x[i];
          const float mean = head_sum(sm) * (EXACT ? 1.0f / DMAX : p.inv_d);
          float c[E], ss = 0.0f;
#pragma unroll
          for (int i = 0; i < E; ++i) {
            c[i] = in_head ? x[i] - mean : 0.0f;
            ss = fmaf(c[i], c[i], ss);
          }
          ss = head_sum(ss);
          const float r = __builtin_amdgcn_rsqf(fmaf(ss, EXACT ? 1.0f / DMAX : p.inv_d, p.eps));
#pragma unroll
          for (int w = 0; w < NV; ++w) {
            float w0, w1, b0, b1;
            IO::unpack(isk[u] ? wk_p.w[w] : wq_p.w[w], w0, w1);
            IO::unpack(isk[u] ? bk_p.w[w] : bq_p.w[w], b0, b1);
            n[2 * w] = fmaf(c[2 * w] * r, w0, b0);
            n[2 * w + 1] = fmaf(c[2 * w + 1] * r, w1, b1);
          }
        } else if constexpr (kRms) {
          float ss = 0.0f;
#pragma unroll
          for (int i = 0; i < E; ++i) ss = fmaf(x[i], x[i], ss);
          ss = head_sum(ss);
          const float r = __builtin_amdgcn_rsqf(fmaf(ss, EXACT ? 1.0f / DMAX : p.inv_d, p.eps));
#pragma unroll
          for (int w = 0; w < NV; ++w) {
            float w0, w1;
            IO::unpack(isk[u] ? wk_p.w[w] : wq_p.w[w], w0, w1);
            n[2 * w] = x[2 * w] * r * w0;
            n[2 * w + 1] = x[2 * w + 1] * r * w1;
          }
        } else {
#pragma unroll
          for (int i = 0; i < E; ++i) n[i] = x[i];
        }
        float o[E];
        if constexpr (!kRotate) {
#pragma unroll
          for (int i = 0; i < E; ++i) o[i] = n[i];
        } else if constexpr (kShift26) {
          // R = 16m + 2*SHIFT ends on slot 4 of a lane: each run of 4 slots is
          // rotated as a whole or passed through
          float* const xrow = shift_rows + wib * kShiftRow;
          wave_lds_fence();  // the previous group's reads are done
          *reinterpret_cast<float4*>(xrow + lane * E) = make_float4(n[0], n[1], n[2], n[3]);
          *reinterpret_cast<float4*>(xrow + lane * E + 4) = make_float4(n[4], n[5], n[6], n[7]);
          wave_lds_fence();
#pragma unroll
          for (int q2 = 0; q2 < E / 2; ++q2) {
            const float2 pn = *reinterpret_cast<const float2*>(xrow + pidx[q2]);
            const int i = 2 * q2;
            const float v0 = fmaf(n[i], cs[i], pn.x * sn[i]);
            const float v1 = fmaf(n[i + 1], cs[i + 1], pn.y * sn[i + 1]);
            o[i] = (FULL || ro_26[i >> 2]) ? v0 : n[i];
            o[i + 1] = (FULL || ro_26[i >> 2]) ? v1 : n[i + 1];
          }
        } else if constexpr (SHIFT == 4) {
#pragma unroll
          for (int i = 0; i < E; ++i) {
            const float pn = lane_fetch(pa_s[i >> 2], n[(i + 4) & 7]);
            const float v = fmaf(n[i], cs[i], pn * sn[i]);
            o[i] = (FULL || ro_s) ? v : n[i];
          }
        } else if constexpr (NEOX) {
#pragma unroll
          for (int i = 0; i < E; ++i) {
            const float pn = lane_fetch(partner_addr, n[i]);
            const float v = fmaf(n[i], cs[i], pn * sn[i]);
            o[i] = lane_rot ? v : n[i];
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < E / 2; ++kk) {
            const float a = n[2 * kk], b = n[2 * kk + 1];
            const float oa = fmaf(a, cs[kk], -(b * sn[kk]));
            const float ob = fmaf(b, cs[kk], a * sn[kk]);
            const bool rot = FULL || (d0 + 2 * kk < R);
            o[2 * kk] = rot ? oa : a;
            o[2 * kk + 1] = rot ? ob : b;
          }
        }
        Raw<NV> out;
#pragma unroll
        for (int w = 0; w < NV; ++w) out.w[w] = IO::pack(o[2 * w], o[2 * w + 1]);
        if (ok[u]) store_io<NV>(rs[u], off[u], out);
      }
    }
  }
}

// ==== fused-kernel device code end

// ----------------------------------------------------------------------------
// Element-granular kernel: the shapes and layouts the vectorised kernel above
// cannot take (head_dims that are not multiples of 8, odd NeoX halves,
// pointers or strides aligned to less than 16 bytes, head strides beyond
// 32-bit lane offsets). Same operation, same fp32 formulas and FMA forms,
// same rounding; only the order of the sums differs.
//
// Lane mapping. A lane slot holds a run of PW consecutive elements (PW = 1, 2,
// 4 or 8: 2-, 4-, 8- or 16-byte accesses); PW divides head_dim and every
// pointer and used stride is 2*PW-byte aligned (the host picks PW). A head
// takes L lanes and S slots per lane (L*S*PW >= head_dim): element e of a head
// sits in lane-in-head (e / PW) % L, slot e / (L*PW). A wave instruction covers
// a head group of G = 64 / L heads of Q, or of K, of one token (G = 1 and
// L up to 64 for large heads), so a group's base address is wave-uniform and
// each lane adds a 32-bit offset (the host checks that a group's offsets fit,
// else it plans one head per group, whose 64-bit base has no stride limit).
// L is a power of two (sum over the head's lanes by DPP steps) or, when that
// fits more heads into a wave instruction, head_dim/(S*PW) rounded up (exact
// fit: a ds_bpermute tree toward the head's first lane plus a broadcast); the
// lanes past the last head of a group and the elements past head_dim take lane
// offsets outside their descriptor's range (loads read zeros, stores are
// dropped), so no access is guarded by a branch. Interleaved partners
// (e, e ^ 1) lie in one run when PW >= 2; NeoX partners (e, e +- R/2), and
// interleaved ones when PW = 1, can sit in any lane and slot, so the
// normalised values of a group go through a per-wave LDS row (G heads x
// L*S*PW floats, head-major) and each element reads its partner.
// A work item is a run of head groups of one token; 16/(S*PW) groups are
// loaded before the first is computed, so every instance keeps 16 elements per
// lane in flight whatever its head_dim.
// ----------------------------------------------------------------------------
constexpr int kElemPerLane = 8;            // S * PW at most
constexpr int kElemMaxDim = 512;
constexpr int kElemRowPad = 12;            // LDS floats per wave after the cos|sin row
// Lane offsets at or past this value lie outside every descriptor's range (the
// host keeps real offsets below 2^31): such loads return zeros without touching
// memory and such stores are dropped.
constexpr uint32_t kElemOob = 0x80000000u;

struct ElemParams {
  int64_t q_tok, k_tok;          // token strides (bytes)
  int64_t q_grp, k_grp;          // bytes between consecutive head groups (G head strides)
  uint32_t q_head, k_head;       // head strides inside a group (0 with G = 1)
  int32_t Hq, Hkv, ngq, ng;      // heads; Q head groups per token (K groups follow); groups per token
  int32_t D, R;
  float inv_d, eps;
  int32_t neox, pos64, has_bias;
  int32_t cs2;                   // cos|sin table 8-byte aligned (rows copied as float2)
  int32_t L, G, seg;             // lanes per head, heads per wave instruction, L not a power of two
  int32_t gpi, nc, n_items;      // groups per item, items per token, items
};

// one I/O element <-> fp32 (the low half of the packed conversions above)
template <class IO>
__device__ __forceinline__ float widen1(uint32_t bits) {
  float lo, hi;
  IO::unpack(bits, lo, hi);
  return lo;
}

template <class IO>
__device__ __forceinline__ uint32_t narrow1(float v) {
  return IO::pack(v, 0.0f) & 0xffffu;
}

// A run of PW elements kept as NW packed dwords (PW = 1: the low half of one).
template <int PW>
struct Run {
  static constexpr int NW = PW >= 2 ? PW / 2 : 1;
  uint32_t w[NW];
};

template <class IO, int PW>
__device__ __forceinline__ void unpack_run(const Run<PW>& r, float* v) {
  if constexpr (PW == 1) {
    v[0] = widen1<IO>(r.w[0]);
  } else {
#pragma unroll
    for (int i = 0; i < PW / 2; ++i) IO::unpack(r.w[i], v[2 * i], v[2 * i + 1]);
  }
}

template <class IO, int PW>
__device__ __forceinline__ Run<PW> pack_run(const float* v) {
  Run<PW> r;
  if constexpr (PW == 1) {
    r.w[0] = narrow1<IO>(v[0]);
  } else {
#pragma unroll
    for (int i = 0; i < PW / 2; ++i) r.w[i] = IO::pack(v[2 * i], v[2 * i + 1]);
  }
  return r;
}

template <int PW, int POLICY>
__device__ __forceinline__ Run<PW> load_run(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  Run<PW> r;
  if constexpr (PW == 8) {
    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, POLICY));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (PW == 4) {
    const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, POLICY));
    r.w[0] = v.x; r.w[1] = v.y;
  } else if constexpr (PW == 2) {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, POLICY);
  } else {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, POLICY);
  }
  return r;
}

template <int PW, int POLICY>
__device__ __forceinline__ void store_run(__amdgpu_buffer_rsrc_t rs, uint32_t off, const Run<PW>& r) {
  if constexpr (PW == 8) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{r.w[0], r.w[1], r.w[2], r.w[3]}, rs, off, 0, POLICY);
  } else if constexpr (PW == 4) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{r.w[0], r.w[1]}, rs, off, 0, POLICY);
  } else if constexpr (PW == 2) {
    __builtin_amdgcn_raw_buffer_store_b32(r.w[0], rs, off, 0, POLICY);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(r.w[0]), rs, off, 0, POLICY);
  }
}

// Sum over aligned groups of L lanes, L a power of two chosen at run time
// (wave-uniform): the steps of group_sum<L> taken while they stay inside a
// group. Every lane of a group gets the same bits.
__device__ __forceinline__ float group_sum_rt(float v, int L) {
  if (L >= 2) v += dpp_mov<kDppQuadXor1>(v);
  if (L >= 4) v += dpp_mov<kDppQuadXor2>(v);
  if (L >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if (L >= 16) v += dpp_mov<kDppRowMirror>(v);
  if (L >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
  if (L == 64) {
    v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  }
  return v;
}

template <class IO, int MODE, int S, int PW>
__global__ void __launch_bounds__(kMaxBlockWaves * kWave)
qknr_elem_kernel(char* __restrict__ qb, char* __restrict__ kb, const void* __restrict__ wqp,
                 const void* __restrict__ wkp, const float* __restrict__ cache,
                 const void* __restrict__ posp, const void* __restrict__ bqp,
                 const void* __restrict__ bkp, const ElemParams p) {
  static_assert(PW == 1 || PW == 2 || PW == 4 || PW == 8, "elements per lane slot");
  static_assert(S >= 1 && S * PW <= kElemPerLane, "at most 8 elements per lane");
  constexpr int NE = S * PW;                  // elements per lane
  constexpr int U = 2 * kElemPerLane / NE;    // groups loaded before the first is computed
  constexpr bool kRotate = MODE == kFused || MODE == kRopeOnly || MODE == kLayerRope;
  constexpr bool kRms = MODE == kFused || MODE == kNormOnly;
  constexpr bool kLayer = MODE == kLayerRope || MODE == kLayerOnly;
  // Runs narrower than 16 bytes leave several wave instructions (slots, or
  // neighbouring head groups) touching one cache line; those loads keep the
  // default policy so the line stays in the caches between them (nontemporal
  // loads there measured 6-19% slower), 16-byte runs stream nontemporally
  constexpr int kElemLoadPolicy = PW == 8 ? kLoadPolicy : 0;
  // Likewise stores of 2 or 4 bytes are left to merge in the L2 (default
  // policy) rather than written through one by one: written through, the
  // 4-byte stores of head_dim 130 wrote 1.43x the stored bytes (default policy
  // there: +29%); 8-byte stores keep the streaming policy (default: -5%)
  constexpr int kElemStorePolicy = PW <= 2 ? 0 : kStorePolicy;
  // The LayerNorm sibling's 16-byte instances lay the token's cos and signed
  // sin out once per item as a pair per element of a head, read back as
  // vectors: no per-element column, sign or rotation flag is kept across the
  // item loop, where that instance is short of scalar registers (+7 to +9% at
  // head_dim 40/38, 128/26, 72/70 and 200/98; the fused op's instances and the
  // narrower ones lost 1-9% with it).
  constexpr bool kPairs = MODE == kLayerRope && PW == 8;
  // per wave: the partner-exchange row (kWave * NE floats) and, with a
  // rotation, the token's cos|sin row (kElemMaxDim floats) and kElemRowPad
  // floats: -0.0f, then a discard area for the runs that hold no element;
  // with kPairs then the pairs (2 * head_dim floats, rounded up to 4)
  extern __shared__ float elem_rows[];
  constexpr int kNegZero = kWave * NE + kElemMaxDim;  // indices into the wave's row
  constexpr int kDiscard = kNegZero + 4;
  constexpr int kPairRow = kNegZero + kElemRowPad;
  const int row_floats = kWave * NE + (kRotate ? kElemMaxDim + kElemRowPad : 0) +
                         (kPairs ? (2 * p.D + 3) & ~3 : 0);
  const int lane = threadIdx.x & (kWave - 1);
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  const int L = p.L, G = p.G;
  const int sub = lane / L;       // head slot in the group
  const int li = lane - sub * L;  // lane inside the head
  const bool in_grp = sub < G;
  const int D = p.D, R = p.R, half = R / 2;
  const bool neox = p.neox != 0;  // wave-uniform
  // partners through LDS: NeoX pairing, or interleaved pairs split over lanes
  const bool exch = kRotate && (neox || PW == 1);
  float* const xrow = elem_rows + wib * row_floats;
  float* const csrow = xrow + kWave * NE;
  const int head0 = sub * (L * NE);  // this head's first element in the row

  // Run s of this lane: elements e0[s] .. e0[s] + PW - 1, all in the head or
  // none (head_dim is a multiple of PW). A run outside the head, or in a lane
  // past the group's last head slot, takes a lane offset outside every
  // descriptor's range: its loads return zeros and its stores are dropped, so
  // no access needs a branch. Its normalised values go to the discard area of
  // the row.
  int e0[S];
  uint32_t qo[S], ko[S];
  int widx[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    e0[s] = (s * L + li) * PW;
    const bool ok = in_grp && e0[s] < D;
    qo[s] = ok ? static_cast<uint32_t>(sub) * p.q_head + 2u * static_cast<uint32_t>(e0[s]) : kElemOob;
    ko[s] = ok ? static_cast<uint32_t>(sub) * p.k_head + 2u * static_cast<uint32_t>(e0[s]) : kElemOob;
    widx[s] = ok ? head0 + e0[s] : kDiscard;
  }
  // where each element reads its partner in the row: the partner's slot for a
  // rotated element, else the -0.0f slot (with cos 1 and sin +0 the rotation
  // then returns the normalised value itself, signed zeros and non-finite
  // values included)
  int pidx[NE];
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int e = e0[s] + i;
      const bool rot = kRotate && in_grp && e < R;
      const int pe = neox ? (e < half ? e + half : e - half) : (e ^ 1);
      pidx[s * PW + i] = rot ? head0 + pe : kNegZero;
    }
  }
  if constexpr (kRotate) {
    if (lane == 0) xrow[kNegZero] = -0.0f;  // ordered before its reads by the fences below
  }

  auto head_sum = [&](float v) { return p.seg ? seg_sum(v, lane, li, L) : group_sum_rt(v, L); };

  // weights and biases of this lane's runs, kept packed; loaded once, after
  // the first head loads are in flight, through descriptors whose range is
  // the row (no bias: an empty range), so runs past head_dim read zeros
  Run<PW> wq[S], wk[S], bq[S], bk[S];
  bool have_w = false;
  auto load_weights = [&]() {
    const uint32_t wrec = static_cast<uint32_t>(2 * D);
    const uint32_t brec = p.has_bias ? wrec : 0u;
    const __amdgpu_buffer_rsrc_t rwq = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wqp), 0, wrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rwk = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(wkp), 0, wrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rbq = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(bqp), 0, brec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rbk = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(bkp), 0, brec, kBufferFlags);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t wo = 2u * static_cast<uint32_t>(e0[s]);
      if constexpr (kRms || kLayer) {
        wq[s] = load_run<PW, 0>(rwq, wo);
        wk[s] = load_run<PW, 0>(rwk, wo);
      }
      if constexpr (kLayer) {
        bq[s] = load_run<PW, 0>(rbq, wo);
        bk[s] = load_run<PW, 0>(rbk, wo);
      }
    }
  };

  const int total_waves = gridDim.x * wpb;
  for (int item = blockIdx.x * wpb + wib; item < p.n_items; item += total_waves) {
    const int t = item / p.nc;
    const int g_begin = (item - t * p.nc) * p.gpi;
    const int g_end = min(g_begin + p.gpi, p.ng);
    char* const qrow = qb + t * p.q_tok;
    char* const krow = kb + t * p.k_tok;

    Run<PW> raw[U][S];
    __amdgpu_buffer_rsrc_t rs[U];
    bool isk[U];
    // a group's descriptor spans its heads that exist (the last group of Q or
    // K may hold fewer than G): lanes of the missing heads fall outside it
    auto issue = [&](int g) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int gu = g + u;
        isk[u] = gu >= p.ngq;  // wave-uniform
        if (gu >= g_end) continue;
        const int gg = isk[u] ? gu - p.ngq : gu;
        const int nvalid = min(G, (isk[u] ? p.Hkv : p.Hq) - gg * G);
        const uint32_t rec = static_cast<uint32_t>(nvalid - 1) * (isk[u] ? p.k_head : p.q_head) +
                             static_cast<uint32_t>(2 * D);
        rs[u] = __builtin_amdgcn_make_buffer_rsrc(isk[u] ? krow + gg * p.k_grp : qrow + gg * p.q_grp,
                                                  0, rec, kBufferFlags);
#pragma unroll
        for (int s = 0; s < S; ++s)
          raw[u][s] = load_run<PW, kElemLoadPolicy>(rs[u], isk[u] ? ko[s] : qo[s]);
      }
    };
    issue(g_begin);
    __builtin_amdgcn_sched_barrier(0);  // the head loads leave first
    if (!have_w) {
      load_weights();
      have_w = true;
    }

    // cos / sin of this lane's elements at this token, the sign of the
    // partner term folded into sin; cos 1 and sin +0 where nothing rotates
    float cs[NE], sn[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      cs[j] = 1.0f;
      sn[j] = 0.0f;
    }
    if constexpr (kRotate) {
      // the wave copies the token's row into LDS with coalesced 8-byte loads
      // (4-byte ones when the table is only 4-byte aligned), then each lane
      // reads the columns of its own elements from there (column 0 where
      // nothing rotates, so every read is in the row)
      const float* const crow = cache + token_position(posp, p.pos64, t) * R;
      wave_lds_fence();  // the previous item's reads of the row are done
      if (p.cs2) {
        for (int c = 2 * lane; c < R; c += 2 * kWave)
          *reinterpret_cast<float2*>(csrow + c) = *reinterpret_cast<const float2*>(crow + c);
      } else {
        for (int c = lane; c < R; c += kWave) csrow[c] = crow[c];
      }
      wave_lds_fence();
      if constexpr (kPairs) {
        // pair e: (cos, -sin) for the first element of a rotation pair,
        // (cos, +sin) for the second, (1, +0) past rope_dim
        float* const prow = xrow + kPairRow;
        for (int e = lane; e < D; e += kWave) {
          float c = 1.0f, v = 0.0f;
          if (e < R) {
            const int col = neox ? (e < half ? e : e - half) : e >> 1;
            c = csrow[col];
            v = csrow[half + col];
            if (neox ? e < half : (e & 1) == 0) v = -v;
          }
          *reinterpret_cast<float2*>(prow + 2 * e) = make_float2(c, v);
        }
        wave_lds_fence();
        // runs past head_dim (and lanes past the last head) read pair 0
        const float* const src = prow + (in_grp && e0[0] < D ? 2 * e0[0] : 0);
#pragma unroll
        for (int i = 0; i < PW; i += 2) {
          const float4 v = *reinterpret_cast<const float4*>(src + 2 * i);
          cs[i] = v.x;
          sn[i] = v.y;
          cs[i + 1] = v.z;
          sn[i + 1] = v.w;
        }
      } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
#pragma unroll
          for (int i = 0; i < PW; ++i) {
            const int j = s * PW + i;
            const int e = e0[s] + i;
            const bool rot = in_grp && e < R;
            const int col = rot ? (neox ? (e < half ? e : e - half) : e >> 1) : 0;
            const bool neg = neox ? e < half : (e & 1) == 0;
            const float c = csrow[col];
            const float v = csrow[half + col];
            cs[j] = rot ? c : 1.0f;
            sn[j] = rot ? (neg ? -v : v) : 0.0f;
          }
        }
      }
    }

    for (int g = g_begin; g < g_end; g += U) {
      if (g != g_begin) issue(g);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (g + u >= g_end) continue;  // wave-uniform: every lane takes part below
        float x[NE];
#pragma unroll
        for (int s = 0; s < S; ++s) unpack_run<IO, PW>(raw[u][s], &x[s * PW]);
        float n[NE];
        if constexpr (kLayer) {
          float sm = 0.0f;
#pragma unroll
          for (int j = 0; j < NE; ++j) sm += x[j];
          const float mean = head_sum(sm) * p.inv_d;
          float c[NE], ss = 0.0f;
#pragma unroll
          for (int j = 0; j < NE; ++j) {
            c[j] = e0[j / PW] < D ? x[j] - mean : 0.0f;  // runs past head_dim add nothing
            ss = fmaf(c[j], c[j], ss);
          }
          ss = head_sum(ss);
          const float r = __builtin_amdgcn_rsqf(fmaf(ss, p.inv_d, p.eps));
#pragma unroll
          for (int s = 0; s < S; ++s) {
            float w[PW], b[PW];
            unpack_run<IO, PW>(isk[u] ? wk[s] : wq[s], w);
            unpack_run<IO, PW>(isk[u] ? bk[s] : bq[s], b);
#pragma unroll
            for (int i = 0; i < PW; ++i) n[s * PW + i] = fmaf(c[s * PW + i] * r, w[i], b[i]);
          }
        } else if constexpr (kRms) {
          float ss = 0.0f;
#pragma unroll
          for (int j = 0; j < NE; ++j) ss = fmaf(x[j], x[j], ss);
          ss = head_sum(ss);
          const float r = __builtin_amdgcn_rsqf(fmaf(ss, p.inv_d, p.eps));
#pragma unroll
          for (int s = 0; s < S; ++s) {
            float w[PW];
            unpack_run<IO, PW>(isk[u] ? wk[s] : wq[s], w);
#pragma unroll
            for (int i = 0; i < PW; ++i) n[s * PW + i] = x[s * PW + i] * r * w[i];
          }
        } else {
#pragma unroll
          for (int j = 0; j < NE; ++j) n[j] = x[j];
        }

        float o[NE];
#pragma unroll
        for (int j = 0; j < NE; ++j) o[j] = n[j];
        if constexpr (kRotate) {
          float pn[NE];
          if (exch) {
            wave_lds_fence();  // the previous group's reads are done
#pragma unroll
            for (int s = 0; s < S; ++s) {
              float* const dst = xrow + widx[s];
              if constexpr (PW == 8) {
                *reinterpret_cast<float4*>(dst) = make_float4(n[s * PW], n[s * PW + 1], n[s * PW + 2], n[s * PW + 3]);
                *reinterpret_cast<float4*>(dst + 4) =
                    make_float4(n[s * PW + 4], n[s * PW + 5], n[s * PW + 6], n[s * PW + 7]);
              } else if constexpr (PW == 4) {
                *reinterpret_cast<float4*>(dst) = make_float4(n[s * PW], n[s * PW + 1], n[s * PW + 2], n[s * PW + 3]);
              } else if constexpr (PW == 2) {
                *reinterpret_cast<float2*>(dst) = make_float2(n[s * PW], n[s * PW + 1]);
              } else {
                *dst = n[s];
              }
            }
            wave_lds_fence();
#pragma unroll
            for (int j = 0; j < NE; ++j) pn[j] = xrow[pidx[j]];
          } else {
            if constexpr (PW >= 2) {
              // interleaved pairs inside a run (R even, runs start at even
              // elements): element e rotates iff e < R
#pragma unroll
              for (int s = 0; s < S; ++s) {
#pragma unroll
                for (int i = 0; i < PW; ++i) {
                  const int j = s * PW + i;
                  pn[j] = e0[s] < R - i ? n[j ^ 1] : -0.0f;
                }
              }
            } else {
#pragma unroll
              for (int j = 0; j < NE; ++j) pn[j] = -0.0f;  // PW = 1 always exchanges
            }
          }
#pragma unroll
          for (int j = 0; j < NE; ++j) o[j] = fmaf(n[j], cs[j], pn[j] * sn[j]);
        }
#pragma unroll
        for (int s = 0; s < S; ++s)
          store_run<PW, kElemStorePolicy>(rs[u], isk[u] ? ko[s] : qo[s], pack_run<IO, PW>(&o[s * PW]));
      }
    }
  }
}

// ----------------------------------------------------------------------------
// One instance group of the kernel table, defined in qknr_inst.hip and built
// once per (I/O type, group): group 0 the fused op with compile-time head_dim,
// group 1 the other modes with compile-time head_dim, groups 2 and 4 the fused
// op and the LayerNorm sibling with a run-time head_dim at unroll 2 and 4 (D is
// then the lane-group capacity). shift 2, 4 or 6 selects the NeoX instances whose
// partners sit that many slots over (fused op, 8 elements per lane). Returns the kernel's host
// stub, or nullptr if no instance matches.
template <class IO, int GROUP>
const void* pick_group(int D, int E, bool neox, bool full, int U, int mode, int shift);

// Groups 2 and 4 (unroll 2 and 4): the fused op and the LayerNorm sibling
// with exact-fit lane groups (SEG) of a run-time head_dim whose NeoX partners
// sit 2 or 6 slots over; nullptr elsewhere.
template <class IO, int GROUP>
const void* pick_seg(bool full, int U, int mode, int shift);

// Groups 3 and 5: the element-granular kernel of a mode (kFused ... kLayerOnly)
// with S slots per lane of pw elements each (pw 1, 2, 4 or 8; S * pw <= 8);
// group 3 holds pw 1 and 2, group 5 pw 4 and 8.
template <class IO, int GROUP>
const void* pick_elem(int mode, int slots, int pw);

}  // namespace qknr_impl
