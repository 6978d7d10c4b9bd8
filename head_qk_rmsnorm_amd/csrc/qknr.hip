// Fused in-place QK RMSNorm + rotary position embedding for MI355X (gfx950).
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
//     is wave-uniform and read with a scalar load (prefetched one item ahead);
//     each lane loads the cos/sin values of its own dims once per item and keeps
//     them in registers for every head of the item.
//   * The fp32 sum of squares is reduced over the L lanes of a head with DPP
//     row operations (quad_perm, row_half_mirror, row_mirror), one ds_swizzle
//     across 16-lane rows for L >= 32 and two readlanes across the wave halves
//     for L = 64; every lane of a head ends with the bit-identical sum.
//   * NeoX partners sit in lane (lane ^ m), m = (rope_dim/2)/E, within the same
//     head; they are fetched with ds_bpermute.
//   * Heads of one token that belong to Q and to K may share a wave
//     instruction: each lane group selects its base pointer, strides and weight
//     row. Only Q/K elements are loaded or stored.
//   * The loads of `unroll` head groups are issued before the first is computed
//     and before the position-dependent cos/sin fetch, so the data is in flight
//     while the position -> cache-row chain resolves. Q/K traffic is streamed
//     with nontemporal loads and stores (each byte is touched once).
//   * By default every wave takes one work item and exits (no persistent grid):
//     the dispatcher back-fills CUs as waves finish, which balances the tail.
// Nothing here is a contraction, so there is no MFMA.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "qknr.h"
#include "qknr_bench.h"

namespace {

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
  } else if constexpr (NV == 2) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    static_assert(NV == 1, "1, 2 or 4 dwords per lane");
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  return r;
}

template <int NV>
__device__ __forceinline__ void store_raw(char* p, const Raw<NV>& r) {
  if constexpr (NV == 4) {
    *reinterpret_cast<u32x4_t*>(p) = u32x4_t{r.w[0], r.w[1], r.w[2], r.w[3]};
  } else if constexpr (NV == 2) {
    *reinterpret_cast<u32x2_t*>(p) = u32x2_t{r.w[0], r.w[1]};
  } else {
    *reinterpret_cast<uint32_t*>(p) = r.w[0];
  }
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

// ----------------------------------------------------------------------------
// Kernel
// ----------------------------------------------------------------------------
// Q/K are read and written exactly once: nontemporal accesses keep them from
// displacing the reused weights, positions and cos|sin rows in L2.
// Q/K accesses go through raw buffer instructions: a wave-uniform descriptor
// (base address of the head group, in SGPRs) plus a 32-bit per-lane offset,
// with the nontemporal cache policy. Offsets stay below 2^31 (checked on the
// host), far inside the descriptor's range, so no access is out of range.
constexpr int kBufferFlags = 0x00020000;  // gfx9 raw-buffer descriptor word 3
constexpr int kCachePolicyNT = 2;          // nontemporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(char* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, kBufferFlags);
}

template <int NV>
__device__ __forceinline__ Raw<NV> load_io(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  Raw<NV> r;
  if constexpr (NV == 4) {
    const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCachePolicyNT));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (NV == 2) {
    const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kCachePolicyNT));
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kCachePolicyNT);
  }
  return r;
}

template <int NV>
__device__ __forceinline__ void store_io(__amdgpu_buffer_rsrc_t rs, uint32_t off, const Raw<NV>& r) {
  if constexpr (NV == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{r.w[0], r.w[1], r.w[2], r.w[3]}, rs, off, 0, kCachePolicyNT);
  } else if constexpr (NV == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{r.w[0], r.w[1]}, rs, off, 0, kCachePolicyNT);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(r.w[0], rs, off, 0, kCachePolicyNT);
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
template <class IO, int DMAX, int E, bool NEOX, bool FULL, int U, int MODE, bool EXACT>
__global__ void __launch_bounds__(kMaxBlockWaves * kWave)
qknr_kernel(char* __restrict__ qb, char* __restrict__ kb, const void* __restrict__ wqp,
            const void* __restrict__ wkp, const float* __restrict__ cache,
            const void* __restrict__ posp, const void* __restrict__ bqp,
            const void* __restrict__ bkp, const Params p) {
  constexpr int L = DMAX / E;   // lanes per head (lane group)
  constexpr int G = kWave / L;  // heads per wave instruction
  constexpr int NV = E / 2;     // packed dwords per lane
  constexpr int NCS = NEOX ? E : E / 2;  // cos (and sin) values per lane
  static_assert(DMAX % E == 0 && E % 2 == 0 && G >= 1, "lane mapping");
  const int lane = threadIdx.x & (kWave - 1);
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  const int sub = lane / L;  // head slot in the group
  const int li = lane % L;   // lane inside the head
  const int d0 = li * E;     // first dim owned by this lane
  const int D = EXACT ? DMAX : p.D;
  const bool in_head = EXACT || d0 < D;  // spare lanes of a run-time head_dim
  const int R = FULL ? D : p.R;
  const int half = R / 2;
  const uint32_t q_off = static_cast<uint32_t>(sub) * p.q_head + d0 * 2;
  const uint32_t k_off = static_cast<uint32_t>(sub) * p.k_head + d0 * 2;

  constexpr bool kRotate = MODE == kFused || MODE == kRopeOnly || MODE == kLayerRope;
  constexpr bool kRms = MODE == kFused || MODE == kNormOnly;
  constexpr bool kLayer = MODE == kLayerRope || MODE == kLayerOnly;

  // Weights (and LayerNorm biases) of this lane's dims, kept packed.
  Raw<NV> wq_p{}, wk_p{}, bq_p{}, bk_p{};
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

  // NeoX: this lane holds dims d0..d0+E-1. With m = (R/2)/E, lanes below m
  // hold first-half dims and find their partners d + R/2 at the same offsets
  // in lane + m; lanes m..2m-1 hold the second half and look m lanes down.
  // Lanes from 2m on hold pass-through dims. Lower-half lanes subtract.
  int partner_addr = lane << 2, j0 = 0;
  bool lower = false, lane_rot = true;
  if constexpr (NEOX) {
    const int m = half / E;
    lane_rot = (FULL && EXACT) || li < 2 * m;
    lower = li < m;
    if (lane_rot) {
      partner_addr = (lower ? lane + m : lane - m) << 2;
      j0 = lower ? d0 : d0 - half;
    }
  } else {
    j0 = in_head ? d0 / 2 : 0;
  }

  const int total_waves = gridDim.x * wpb;
  int item = blockIdx.x * wpb + wib;
  if (item >= p.n_items) return;
  int64_t pos_next = kRotate ? token_position(posp, p.pos64, item / p.nc) : 0;

  for (; item < p.n_items; item += total_waves) {
    const int t = item / p.nc;
    const int g_begin = (item - t * p.nc) * p.gpi;
    const int g_end = min(g_begin + p.gpi, p.ng);
    const int64_t pos = pos_next;
    if (kRotate && item + total_waves < p.n_items)
      pos_next = token_position(posp, p.pos64, (item + total_waves) / p.nc);
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

    // cos / sin of this lane's dims at this token (loaded after the head data
    // is in flight; kept in registers for every group of the item)
    float cs[NCS], sn[NCS];
    if constexpr (kRotate) {
      const float* row = cache + pos * R;
      if ((FULL || NEOX) && NCS % 4 == 0 && p.cs_vec) {
#pragma unroll
        for (int i = 0; i < NCS; i += 4) {
          const float4 c4 = *reinterpret_cast<const float4*>(row + j0 + i);
          const float4 s4 = *reinterpret_cast<const float4*>(row + half + j0 + i);
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
      if constexpr (NEOX) {
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
          const float mean = group_sum<L>(sm) * (EXACT ? 1.0f / DMAX : p.inv_d);
          float c[E], ss = 0.0f;
#pragma unroll
          for (int i = 0; i < E; ++i) {
            c[i] = in_head ? x[i] - mean : 0.0f;
            ss = fmaf(c[i], c[i], ss);
          }
          ss = group_sum<L>(ss);
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
          ss = group_sum<L>(ss);
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
            const bool rot = (FULL && EXACT) || (d0 + 2 * kk < R);
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

// Measurement aids (see qknr_bench.h): one 16-byte element per thread, one
// pass over the grid, nontemporal like the op's Q/K traffic.
__global__ void __launch_bounds__(256) copy_kernel(u32x4_t* __restrict__ dst,
                                                   const u32x4_t* __restrict__ src, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

__global__ void __launch_bounds__(256) rmw_kernel(u32x4_t* buf, int64_t n, uint32_t key) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(&buf[i]);
    __builtin_nontemporal_store(v ^ key, &buf[i]);
  }
}

// ----------------------------------------------------------------------------
// Kernel table
// ----------------------------------------------------------------------------
template <class IO, int D, int E, bool NEOX, bool FULL>
const void* pick_unroll(int U, int mode) {
  if (mode == kFused) {
    switch (U) {
      case 1: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 1, kFused, true>);
      case 2: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 2, kFused, true>);
      case 4: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 4, kFused, true>);
      default: return nullptr;
    }
  }
  // the unfused baseline steps and the LayerNorm sibling exist at unroll 2 only
  if (U != 2) return nullptr;
  if (mode == kRopeOnly)
    return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 2, kRopeOnly, true>);
  if (mode == kLayerRope)
    return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 2, kLayerRope, true>);
  if (!NEOX && FULL) {  // pairing and rope_dim play no part without a rotation
    if (mode == kNormOnly)
      return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, false, true, 2, kNormOnly, true>);
    if (mode == kLayerOnly)
      return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, false, true, 2, kLayerOnly, true>);
  }
  return nullptr;
}

template <class IO, int D, int E>
const void* pick_pairing(bool neox, bool full, int U, int mode) {
  if (neox) return full ? pick_unroll<IO, D, E, true, true>(U, mode) : pick_unroll<IO, D, E, true, false>(U, mode);
  return full ? pick_unroll<IO, D, E, false, true>(U, mode) : pick_unroll<IO, D, E, false, false>(U, mode);
}

// Elements per lane: 8 (16-byte lanes), head_dim/32 (half a wave per head) and
// head_dim/64 (a full wave per head; needs an even count, so not head_dim 64).
template <class IO, int D>
const void* pick_lanes(int E, bool neox, bool full, int U, int mode) {
  if (E == 8) return pick_pairing<IO, D, 8>(neox, full, U, mode);
  if constexpr (D / 32 != 8) {
    if (E == D / 32) return pick_pairing<IO, D, D / 32>(neox, full, U, mode);
  }
  if constexpr (D / 64 >= 2 && D / 64 != 8) {
    if (E == D / 64) return pick_pairing<IO, D, D / 64>(neox, full, U, mode);
  }
  return nullptr;
}

// Run-time head_dim instances: 16-byte lanes, lane group of DMAX/8 lanes, the
// fused op and the LayerNorm sibling at unroll 2.
template <class IO, int DMAX, int MODE>
const void* pick_any_dim_mode(bool neox, bool full) {
  if (neox) {
    return full ? reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, true, true, 2, MODE, false>)
                : reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, true, false, 2, MODE, false>);
  }
  return full ? reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, false, true, 2, MODE, false>)
              : reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, false, false, 2, MODE, false>);
}

template <class IO, int DMAX>
const void* pick_any_dim(bool neox, bool full, int mode) {
  switch (mode) {
    case kFused: return pick_any_dim_mode<IO, DMAX, kFused>(neox, full);
    case kLayerRope: return pick_any_dim_mode<IO, DMAX, kLayerRope>(neox, full);
    case kLayerOnly:
      return reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, false, true, 2, kLayerOnly, false>);
    default: return nullptr;
  }
}

template <class IO>
const void* pick_dim(int D, int E, bool neox, bool full, int U, int mode, bool exact) {
  if (!exact) {
    if (U != 2 || E != 8) return nullptr;
    switch (D) {  // D is the lane-group capacity DMAX here
      case 16: return pick_any_dim<IO, 16>(neox, full, mode);
      case 32: return pick_any_dim<IO, 32>(neox, full, mode);
      case 64: return pick_any_dim<IO, 64>(neox, full, mode);
      case 128: return pick_any_dim<IO, 128>(neox, full, mode);
      case 256: return pick_any_dim<IO, 256>(neox, full, mode);
      case 512: return pick_any_dim<IO, 512>(neox, full, mode);
      default: return nullptr;
    }
  }
  switch (D) {
    case 64: return pick_lanes<IO, 64>(E, neox, full, U, mode);
    case 128: return pick_lanes<IO, 128>(E, neox, full, U, mode);
    case 256: return pick_lanes<IO, 256>(E, neox, full, U, mode);
    default: return nullptr;
  }
}

const void* pick_kernel(int dtype, int D, int E, bool neox, bool full, int U, int mode, bool exact) {
  return dtype == QKNR_BF16 ? pick_dim<Bf16>(D, E, neox, full, U, mode, exact)
                            : pick_dim<Fp16>(D, E, neox, full, U, mode, exact);
}

// ----------------------------------------------------------------------------
// Host-side validation and planning (no HIP call before validation passes)
// ----------------------------------------------------------------------------
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// head_dim with compile-time instances (every lane mapping)
bool fast_head_dim(int32_t D) { return D == 64 || D == 128 || D == 256; }

// other head_dims: multiples of 8 from 16 to 512, run-time instances
bool any_head_dim(int32_t D) { return !fast_head_dim(D) && D % 8 == 0 && D >= 16 && D <= 512; }

// lane-group capacity of a run-time head_dim: the next power of two, >= 16
int any_dim_capacity(int32_t D) {
  int c = 16;
  while (c < D) c *= 2;
  return c;
}

// NeoX pairs (d, d + R/2): with E elements per lane the partner sits a fixed
// m = (R/2)/E lanes away when R/2 is a multiple of E.
bool lanes_fit(int32_t R, int32_t neox, int E) {
  if (!neox) return true;
  return (R / 2) % E == 0 && R / 2 >= E;
}

// The supported set: the page's rule (head_dim 64/128/256, rope_dim a
// multiple of head_dim/32, NeoX rotary lanes a power of two) widened to every
// even rope_dim for interleaved pairing, every NeoX rope_dim whose half is a
// multiple of some lane width, and other head_dims that are multiples of 8.
bool shape_supported(int32_t D, int32_t R, int32_t neox) {
  if (!fast_head_dim(D) && !any_head_dim(D)) return false;
  if (R <= 0 || R > D || R % 2) return false;
  if (!neox) return true;
  if (fast_head_dim(D)) {
    if (lanes_fit(R, neox, 8) || lanes_fit(R, neox, D / 32)) return true;
    return D / 64 >= 2 && lanes_fit(R, neox, D / 64);
  }
  return lanes_fit(R, neox, 8);
}

// Head vectors of one tensor must not overlap: with the smaller of the two
// strides inner, it must cover a vector and the outer one the inner extent.
bool views_ok(int64_t T, int64_t H, int64_t tok, int64_t head, int64_t vec_bytes) {
  if (tok < 0 || head < 0) return false;
  const bool use_t = T > 1, use_h = H > 1;
  if (!use_t && !use_h) return true;
  if (use_t && !use_h) return tok >= vec_bytes;
  if (!use_t && use_h) return head >= vec_bytes;
  int64_t s_in = head, n_in = H, s_out = tok;
  if (tok < head) { s_in = tok; n_in = T; s_out = head; }
  if (s_in < vec_bytes) return false;
  if (n_in > 0 && s_in > INT64_MAX / n_in) return false;
  return s_out >= s_in * n_in;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Launch defaults, chosen by measurement on MI355X (launch-shape sweeps over
// the benchmark workloads): one work item per wave with no persistent grid,
// 2 head groups per item, both loaded before the first is computed, 4 waves
// per workgroup.
constexpr int kDefaultGroupsPerItem = 2;
constexpr int kDefaultUnroll = 2;
constexpr int kDefaultBlockWaves = 4;

struct Plan {
  const void* fn = nullptr;
  int E = 8, L = 8, G = 8, ngq = 0, ng = 0, gpi = 0, nc = 0, U = kDefaultUnroll,
      wpb = kDefaultBlockWaves;
  int64_t items = 0;
  int max_blocks = 0;  // 0: one workgroup per wpb items; -1: occupancy x CUs; > 0: explicit cap
  int dmax = 0;        // head_dim of the instance (lane-group capacity)
  bool exact = true;   // head_dim == dmax
};

// A lane's byte offset inside its head group, (heads-1)*head_stride + 2*D at
// most, must stay below 2^31 (head-major layouts with a huge T can exceed it
// for groups of several heads; a mapping with fewer heads per group is used).
constexpr int64_t kMaxLaneOffset = (int64_t{1} << 31) - 1;

bool lane_offsets_fit(int G, int32_t H, int64_t head_stride, int32_t D) {
  const int64_t heads = std::min<int64_t>(G, H);
  if (heads <= 1) return true;
  if (head_stride < 0 || head_stride > (kMaxLaneOffset - 2 * D) / (heads - 1)) return false;
  return true;
}

int32_t make_plan(int mode, int64_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t R,
                  int32_t neox, int32_t dtype, int64_t q_head, int64_t k_head,
                  const qknr_launch_cfg* cfg, Plan* pl) {
  qknr_launch_cfg c = cfg ? *cfg : qknr_launch_cfg{0, 0, 0, 0, 0};
  auto fits = [&](int E) {
    const int G = kWave / (D / E);
    return lane_offsets_fit(G, Hq, q_head, D) && lane_offsets_fit(G, Hkv, k_head, D);
  };
  int E = 0;
  const bool exact = fast_head_dim(D);
  const int dmax = exact ? D : any_dim_capacity(D);
  if (!exact) {
    // run-time head_dim: 16-byte lanes in a lane group of dmax/8 lanes
    E = 8;
    const int G = kWave / (dmax / 8);
    if (!lanes_fit(R, neox, 8)) return QKNR_E_UNSUPPORTED;
    if (c.lanes_per_head != 0 && c.lanes_per_head != dmax / 8) return QKNR_E_ARG;
    if (!lane_offsets_fit(G, Hq, q_head, D) || !lane_offsets_fit(G, Hkv, k_head, D))
      return QKNR_E_SHAPE;
  } else if (c.lanes_per_head == 0) {
    // 16-byte lanes first; then half a wave and a full wave per head
    const int cand[3] = {8, D / 32, D / 64};
    for (int e : cand) {
      if (e >= 2 && lanes_fit(R, neox, e) && fits(e)) { E = e; break; }
    }
    if (E == 0) return QKNR_E_SHAPE;
  } else {
    if (c.lanes_per_head <= 0 || c.lanes_per_head > kWave || D % c.lanes_per_head != 0)
      return QKNR_E_ARG;
    E = D / c.lanes_per_head;
    if (E != 8 && E != D / 32 && !(E == D / 64 && E >= 2)) return QKNR_E_ARG;
    if (!lanes_fit(R, neox, E) || !fits(E)) return QKNR_E_ARG;
  }
  // the unfused baseline steps and the run-time head_dim instances exist at unroll 2 only
  const int U = (mode != kFused || !exact) ? 2 : (c.unroll == 0 ? kDefaultUnroll : c.unroll);
  if (U != 1 && U != 2 && U != 4) return QKNR_E_ARG;
  const int wpb = c.block_waves == 0 ? kDefaultBlockWaves : c.block_waves;
  if (wpb < 1 || wpb > kMaxBlockWaves) return QKNR_E_ARG;
  if (c.groups_per_item < 0 || c.max_blocks < -1) return QKNR_E_ARG;

  pl->E = E;
  pl->L = dmax / E;
  pl->dmax = dmax;
  pl->exact = exact;
  pl->G = kWave / pl->L;
  pl->ngq = (Hq + pl->G - 1) / pl->G;
  pl->ng = pl->ngq + (Hkv + pl->G - 1) / pl->G;
  const int want_gpi = c.groups_per_item == 0 ? kDefaultGroupsPerItem : c.groups_per_item;
  pl->gpi = std::max(1, std::min(want_gpi, pl->ng));
  pl->nc = (pl->ng + pl->gpi - 1) / pl->gpi;
  pl->items = T * pl->nc;
  if (pl->items > INT32_MAX) return QKNR_E_SHAPE;
  pl->U = U;
  pl->wpb = wpb;
  pl->max_blocks = c.max_blocks;
  pl->fn = pick_kernel(dtype, dmax, E, neox != 0, R == D, U, mode, exact);
  return pl->fn ? QKNR_OK : QKNR_E_UNSUPPORTED;
}

// Per-device CU count and per-kernel occupancy, computed once.
std::mutex g_cache_mu;
std::map<int, int> g_cus;
std::map<std::pair<const void*, int>, int> g_occ;

int32_t device_limits(const void* fn, int threads, size_t lds, int* cus, int* blocks_per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QKNR_E_DEVICE;
  std::lock_guard<std::mutex> lk(g_cache_mu);
  auto it = g_cus.find(dev);
  if (it == g_cus.end()) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return QKNR_E_DEVICE;
    it = g_cus.emplace(dev, n).first;
  }
  *cus = it->second;
  auto key = std::make_pair(fn, threads);
  auto jt = g_occ.find(key);
  if (jt == g_occ.end()) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, lds) != hipSuccess || nb <= 0)
      nb = 1;
    jt = g_occ.emplace(key, nb).first;
  }
  *blocks_per_cu = jt->second;
  return QKNR_OK;
}

// One call of the op or of one unfused step, with every argument.
struct Call {
  void* q;
  void* k;
  const void* wq;
  const void* wk;
  const float* cache;
  const void* pos;
  const void* bq;  // LayerNorm biases (NULL: none)
  const void* bk;
  int64_t T;
  int32_t Hq, Hkv, D, R, neox;
  float eps;
  int64_t qt, qh, kt, kh;  // byte strides
  int32_t dtype, pdt;
  hipStream_t stream;
};

// Validation (no HIP call) and planning. For kNormOnly the rotation arguments
// are ignored (pass rope_dim = head_dim); for kRopeOnly the weights and eps.
int32_t prepare(int mode, const Call& c, const qknr_launch_cfg* cfg, Plan* pl,
                qknr_launch_info* info) {
  if (c.T < 0 || c.Hq < 0 || c.Hkv < 0) return QKNR_E_SHAPE;
  if (c.dtype != QKNR_BF16 && c.dtype != QKNR_FP16) return QKNR_E_DTYPE;
  if (c.pdt != QKNR_I32 && c.pdt != QKNR_I64) return QKNR_E_DTYPE;
  if (!shape_supported(c.D, c.R, c.neox)) return QKNR_E_UNSUPPORTED;
  if (!std::isfinite(c.eps) || c.eps < 0.0f) return QKNR_E_ARG;
  if (c.T > INT32_MAX || c.T * (static_cast<int64_t>(c.Hq) + c.Hkv) > INT32_MAX) return QKNR_E_SHAPE;

  const int32_t prc = make_plan(mode, c.T, c.Hq, c.Hkv, c.D, c.R, c.neox, c.dtype, c.qh, c.kh, cfg, pl);
  if (prc != QKNR_OK) return prc;
  if (info) {
    info->lanes_per_head = pl->L;
    info->elems_per_lane = pl->E;
    info->heads_per_wave = pl->G;
    info->groups_per_token = pl->ng;
    info->groups_per_item = pl->gpi;
    info->unroll = pl->U;
    info->block_threads = pl->wpb * kWave;
    info->grid_blocks = 0;
    info->items = pl->items;
  }
  if (c.T == 0 || c.Hq + c.Hkv == 0) return QKNR_OK;

  const bool need_w = mode != kRopeOnly;
  const bool need_rot = mode == kFused || mode == kRopeOnly || mode == kLayerRope;
  const bool bias = (mode == kLayerRope || mode == kLayerOnly) && (c.bq || c.bk);
  if ((c.Hq > 0 && (!c.q || (need_w && !c.wq) || (bias && !c.bq))) ||
      (c.Hkv > 0 && (!c.k || (need_w && !c.wk) || (bias && !c.bk))) ||
      (need_rot && (!c.cache || !c.pos)))
    return QKNR_E_NULL;
  if (bias && ((c.bq && !aligned(c.bq, 16)) || (c.bk && !aligned(c.bk, 16)))) return QKNR_E_ALIGN;
  const int64_t vec = 2 * static_cast<int64_t>(c.D);
  if (c.Hq > 0 && !views_ok(c.T, c.Hq, c.qt, c.qh, vec)) return QKNR_E_SHAPE;
  if (c.Hkv > 0 && !views_ok(c.T, c.Hkv, c.kt, c.kh, vec)) return QKNR_E_SHAPE;
  if (c.Hq > 0 && (!aligned(c.q, 16) || (need_w && !aligned(c.wq, 16)) || (c.T > 1 && c.qt % 16) ||
                   (c.Hq > 1 && c.qh % 16)))
    return QKNR_E_ALIGN;
  if (c.Hkv > 0 && (!aligned(c.k, 16) || (need_w && !aligned(c.wk, 16)) || (c.T > 1 && c.kt % 16) ||
                    (c.Hkv > 1 && c.kh % 16)))
    return QKNR_E_ALIGN;
  if (need_rot && (!aligned(c.cache, 4) || !aligned(c.pos, c.pdt == QKNR_I64 ? 8 : 4)))
    return QKNR_E_ALIGN;
  return QKNR_OK;
}

// Enqueue a prepared call (HIP calls from here on).
int32_t launch(const Call& c, const Plan& pl, qknr_launch_info* info) {
  if (c.T == 0 || c.Hq + c.Hkv == 0) return QKNR_OK;
  const int threads = pl.wpb * kWave;
  int cus = 0, per_cu = 0;
  const int32_t drc = device_limits(pl.fn, threads, 0, &cus, &per_cu);
  if (drc != QKNR_OK) return drc;
  const int64_t needed = (pl.items + pl.wpb - 1) / pl.wpb;
  int64_t cap = needed;
  if (pl.max_blocks > 0) cap = pl.max_blocks;
  if (pl.max_blocks == -1) cap = static_cast<int64_t>(cus) * per_cu;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min(needed, cap)));
  if (info) info->grid_blocks = grid;

  Params prm;
  char* qarg = static_cast<char*>(c.q);
  char* karg = static_cast<char*>(c.k);
  const void* wqarg = c.wq ? c.wq : c.wk;  // the side with 0 heads still gets a readable row
  const void* wkarg = c.wk ? c.wk : c.wq;
  const float* carg = c.cache;
  const void* parg = c.pos;
  const void* bqarg = c.bq ? c.bq : c.bk;  // the side with 0 heads still gets a readable row
  const void* bkarg = c.bk ? c.bk : c.bq;
  prm.has_bias = (c.bq || c.bk) ? 1 : 0;
  prm.cs_vec = (reinterpret_cast<uintptr_t>(c.cache) % 16 == 0) && ((c.R / 2) % 4 == 0);
  // head strides only matter for views with more than one head
  const int64_t qh = c.Hq > 1 ? c.qh : 0, kh = c.Hkv > 1 ? c.kh : 0;
  prm.q_tok = c.qt;
  prm.k_tok = c.kt;
  prm.q_grp = qh * pl.G;
  prm.k_grp = kh * pl.G;
  prm.q_head = static_cast<uint32_t>(qh);
  prm.k_head = static_cast<uint32_t>(kh);
  prm.ngq = pl.ngq;
  prm.Hq = c.Hq;
  prm.Hkv = c.Hkv;
  prm.R = c.R;
  prm.D = c.D;
  prm.inv_d = static_cast<float>(1.0 / c.D);
  prm.pos64 = c.pdt == QKNR_I64;
  prm.eps = c.eps;
  prm.ng = pl.ng;
  prm.gpi = pl.gpi;
  prm.nc = pl.nc;
  prm.n_items = static_cast<int32_t>(pl.items);
  void* args[] = {&qarg, &karg, &wqarg, &wkarg, &carg, &parg, &bqarg, &bkarg, &prm};
  if (hipLaunchKernel(pl.fn, dim3(grid), dim3(threads), args, 0, c.stream) != hipSuccess)
    return QKNR_E_LAUNCH;
  return QKNR_OK;
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------
extern "C" {

QKNR_API int32_t qknr_can_use(int32_t head_dim, int32_t rope_dim, int32_t is_neox, int32_t dtype,
                              int32_t pos_dtype) {
  if (dtype != QKNR_BF16 && dtype != QKNR_FP16) return 0;
  if (pos_dtype != QKNR_I32 && pos_dtype != QKNR_I64) return 0;
  return shape_supported(head_dim, rope_dim, is_neox) ? 1 : 0;
}

QKNR_API const char* qknr_status_string(int32_t status) {
  switch (status) {
    case QKNR_OK: return "ok";
    case QKNR_E_NULL: return "qknr: a required pointer is NULL";
    case QKNR_E_SHAPE: return "qknr: bad shape or strides (negative, overlapping head vectors, or too large)";
    case QKNR_E_UNSUPPORTED:
      return "qknr: unsupported (head_dim, rope_dim, is_neox): need head_dim a multiple of 8 in "
             "[16, 512], rope_dim even in (0, head_dim], and for NeoX rope_dim/2 a multiple of 8 "
             "(for head_dim 64/128/256 a multiple of 2, 2 or 4); the unfused steps take head_dim "
             "64/128/256 only";
    case QKNR_E_ALIGN:
      return "qknr: misaligned: q, k, weights and q/k strides need 16-byte alignment, the cache 4 bytes, "
             "positions their element size";
    case QKNR_E_DTYPE: return "qknr: unknown dtype or pos_dtype code";
    case QKNR_E_ARG: return "qknr: bad argument (eps must be finite and >= 0; launch configuration invalid)";
    case QKNR_E_LAUNCH: return "qknr: the HIP runtime rejected the kernel launch";
    case QKNR_E_DEVICE: return "qknr: could not query the current HIP device";
    default: return "qknr: unknown status";
  }
}

QKNR_API int32_t qknr_inplace_ex(void* q, void* k, const void* wq, const void* wk,
                                 const float* cos_sin_cache, const void* positions, int64_t T,
                                 int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t rope_dim,
                                 int32_t is_neox, float eps, int64_t q_tok_stride_B,
                                 int64_t q_head_stride_B, int64_t k_tok_stride_B,
                                 int64_t k_head_stride_B, int32_t dtype, int32_t pos_dtype,
                                 hipStream_t stream, const qknr_launch_cfg* cfg,
                                 qknr_launch_info* info) {
  const Call c{q, k, wq, wk, cos_sin_cache, positions, nullptr, nullptr, T, Hq, Hkv, head_dim,
               rope_dim, is_neox, eps, q_tok_stride_B, q_head_stride_B, k_tok_stride_B,
               k_head_stride_B, dtype, pos_dtype, stream};
  Plan pl;
  const int32_t rc = prepare(kFused, c, cfg, &pl, info);
  return rc != QKNR_OK ? rc : launch(c, pl, info);
}

QKNR_API int32_t qknr_inplace(void* q, void* k, const void* wq, const void* wk,
                              const float* cos_sin_cache, const void* positions, int64_t T,
                              int32_t Hq, int32_t Hkv, int32_t head_dim, int32_t rope_dim,
                              int32_t is_neox, float eps, int64_t q_tok_stride_B,
                              int64_t q_head_stride_B, int64_t k_tok_stride_B,
                              int64_t k_head_stride_B, int32_t dtype, int32_t pos_dtype,
                              hipStream_t stream) {
  return qknr_inplace_ex(q, k, wq, wk, cos_sin_cache, positions, T, Hq, Hkv, head_dim, rope_dim,
                         is_neox, eps, q_tok_stride_B, q_head_stride_B, k_tok_stride_B,
                         k_head_stride_B, dtype, pos_dtype, stream, nullptr, nullptr);
}

QKNR_API int32_t qknr_rmsnorm_inplace(void* q, void* k, const void* wq, const void* wk, int64_t T,
                                      int32_t Hq, int32_t Hkv, int32_t head_dim, float eps,
                                      int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                      int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                      int32_t dtype, hipStream_t stream) {
  const Call c{q, k, wq, wk, nullptr, nullptr, nullptr, nullptr, T, Hq, Hkv, head_dim, head_dim,
               0, eps, q_tok_stride_B, q_head_stride_B, k_tok_stride_B, k_head_stride_B, dtype,
               QKNR_I32, stream};
  Plan pl;
  const int32_t rc = prepare(kNormOnly, c, nullptr, &pl, nullptr);
  return rc != QKNR_OK ? rc : launch(c, pl, nullptr);
}

QKNR_API int32_t qknr_rope_inplace(void* q, void* k, const float* cos_sin_cache,
                                   const void* positions, int64_t T, int32_t Hq, int32_t Hkv,
                                   int32_t head_dim, int32_t rope_dim, int32_t is_neox,
                                   int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                   int64_t k_tok_stride_B, int64_t k_head_stride_B, int32_t dtype,
                                   int32_t pos_dtype, hipStream_t stream) {
  const Call c{q, k, nullptr, nullptr, cos_sin_cache, positions, nullptr, nullptr, T, Hq, Hkv,
               head_dim, rope_dim, is_neox, 0.0f, q_tok_stride_B, q_head_stride_B, k_tok_stride_B,
               k_head_stride_B, dtype, pos_dtype, stream};
  Plan pl;
  const int32_t rc = prepare(kRopeOnly, c, nullptr, &pl, nullptr);
  return rc != QKNR_OK ? rc : launch(c, pl, nullptr);
}

QKNR_API int32_t qknr_unfused_inplace(void* q, void* k, const void* wq, const void* wk,
                                      const float* cos_sin_cache, const void* positions,
                                      int64_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                      int32_t rope_dim, int32_t is_neox, float eps,
                                      int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                      int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                      int32_t dtype, int32_t pos_dtype, hipStream_t stream) {
  // validate everything for both steps before enqueueing either
  const Call c{q, k, wq, wk, cos_sin_cache, positions, nullptr, nullptr, T, Hq, Hkv, head_dim,
               rope_dim, is_neox, eps, q_tok_stride_B, q_head_stride_B, k_tok_stride_B,
               k_head_stride_B, dtype, pos_dtype, stream};
  Plan fused, norm, rot;
  int32_t rc = prepare(kFused, c, nullptr, &fused, nullptr);
  if (rc != QKNR_OK) return rc;
  Call cn = c;
  cn.R = head_dim;
  cn.neox = 0;
  rc = prepare(kNormOnly, cn, nullptr, &norm, nullptr);
  if (rc != QKNR_OK) return rc;
  rc = prepare(kRopeOnly, c, nullptr, &rot, nullptr);
  if (rc != QKNR_OK) return rc;
  rc = launch(cn, norm, nullptr);
  return rc != QKNR_OK ? rc : launch(c, rot, nullptr);
}

QKNR_API int32_t qknr_layernorm_rope_inplace(void* q, void* k, const void* wq, const void* wk,
                                             const void* bq, const void* bk,
                                             const float* cos_sin_cache, const void* positions,
                                             int64_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                             int32_t rope_dim, int32_t is_neox, float eps,
                                             int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                             int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                             int32_t dtype, int32_t pos_dtype, hipStream_t stream) {
  const bool rotate = rope_dim != 0;
  const Call c{q, k, wq, wk, rotate ? cos_sin_cache : nullptr, rotate ? positions : nullptr, bq, bk,
               T, Hq, Hkv, head_dim, rotate ? rope_dim : head_dim, rotate ? is_neox : 0, eps,
               q_tok_stride_B, q_head_stride_B, k_tok_stride_B, k_head_stride_B, dtype,
               rotate ? pos_dtype : QKNR_I32, stream};
  Plan pl;
  const int32_t rc = prepare(rotate ? kLayerRope : kLayerOnly, c, nullptr, &pl, nullptr);
  return rc != QKNR_OK ? rc : launch(c, pl, nullptr);
}

static int32_t stream_launch(const void* fn, void** args, int64_t n16, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QKNR_E_DEVICE;
  const int64_t needed = (n16 + 255) / 256;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(needed, INT32_MAX)));
  if (hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, stream) != hipSuccess) return QKNR_E_LAUNCH;
  return QKNR_OK;
}

QKNR_API int32_t qknr_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (bytes < 0) return QKNR_E_SHAPE;
  if (bytes == 0) return QKNR_OK;
  if (!dst || !src) return QKNR_E_NULL;
  if (!aligned(dst, 16) || !aligned(src, 16) || bytes % 16) return QKNR_E_ALIGN;
  u32x4_t* d = static_cast<u32x4_t*>(dst);
  const u32x4_t* s = static_cast<const u32x4_t*>(src);
  int64_t n = bytes / 16;
  void* args[] = {&d, &s, &n};
  return stream_launch(reinterpret_cast<const void*>(&copy_kernel), args, n, stream);
}

QKNR_API int32_t qknr_rmw(void* buf, int64_t bytes, uint32_t key, hipStream_t stream) {
  if (bytes < 0) return QKNR_E_SHAPE;
  if (bytes == 0) return QKNR_OK;
  if (!buf) return QKNR_E_NULL;
  if (!aligned(buf, 16) || bytes % 16) return QKNR_E_ALIGN;
  u32x4_t* b = static_cast<u32x4_t*>(buf);
  int64_t n = bytes / 16;
  void* args[] = {&b, &n, &key};
  return stream_launch(reinterpret_cast<const void*>(&rmw_kernel), args, n, stream);
}

}  // extern "C"
