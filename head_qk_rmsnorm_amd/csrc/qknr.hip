// Host library of the fused in-place QK RMSNorm + rotary position embedding for
// MI355X (gfx950): argument validation, launch planning, the C ABI declared in
// include/qknr.h and include/qknr_bench.h, and the two measurement kernels.
// The op's kernels live in qknr_device.h / qknr_inst.hip; the operation is the
// one of the page "SGLang Diffusion fused operator fused_inplace_qknorm_rope:
// in-depth technical analysis" (m.lsln.cn/news/241376), sections 2.1-2.3 and 3.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "qknr.h"
#include "qknr_bench.h"
#include "qknr_device.h"

namespace {

using namespace qknr_impl;

// Measurement aids (see qknr_bench.h): one 16-byte element per thread, one
// pass over the grid, with the op's Q/K cache policies (nontemporal loads;
// nontemporal, agent-scope stores). Each workgroup addresses its own 4 KiB
// chunk through a buffer descriptor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 4096, kBufferFlags);
}

__global__ void __launch_bounds__(256) copy_kernel(char* __restrict__ dst,
                                                   const char* __restrict__ src, int64_t n) {
  for (int64_t blk = blockIdx.x; blk * 256 < n; blk += gridDim.x) {
    if (blk * 256 + threadIdx.x < n) {
      const uint32_t off = threadIdx.x * 16;
      const u32x4_t v = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(chunk_rsrc(src + blk * 4096), off, 0, kLoadPolicy));
      __builtin_amdgcn_raw_buffer_store_b128(v, chunk_rsrc(dst + blk * 4096), off, 0, kStorePolicy);
    }
  }
}

__global__ void __launch_bounds__(256) rmw_kernel(char* buf, int64_t n, uint32_t key) {
  for (int64_t blk = blockIdx.x; blk * 256 < n; blk += gridDim.x) {
    if (blk * 256 + threadIdx.x < n) {
      const uint32_t off = threadIdx.x * 16;
      const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(buf + blk * 4096);
      const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kLoadPolicy));
      __builtin_amdgcn_raw_buffer_store_b128(v ^ key, rs, off, 0, kStorePolicy);
    }
  }
}

const void* pick_kernel(int dtype, int D, int E, bool neox, bool full, int U, int mode, bool exact,
                        int shift) {
  const int group = !exact ? (U == 4 ? 4 : 2) : (mode == kFused ? 0 : 1);
  if (dtype == QKNR_BF16) {
    switch (group) {
      case 0: return pick_group<Bf16, 0>(D, E, neox, full, U, mode, shift);
      case 1: return pick_group<Bf16, 1>(D, E, neox, full, U, mode, shift);
      case 2: return pick_group<Bf16, 2>(D, E, neox, full, U, mode, shift);
      default: return pick_group<Bf16, 4>(D, E, neox, full, U, mode, shift);
    }
  }
  switch (group) {
    case 0: return pick_group<Fp16, 0>(D, E, neox, full, U, mode, shift);
    case 1: return pick_group<Fp16, 1>(D, E, neox, full, U, mode, shift);
    case 2: return pick_group<Fp16, 2>(D, E, neox, full, U, mode, shift);
    default: return pick_group<Fp16, 4>(D, E, neox, full, U, mode, shift);
  }
}

// ----------------------------------------------------------------------------
// Host-side validation and planning (no HIP call before validation passes)
// ----------------------------------------------------------------------------

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

const void* pick_seg_kernel(int dtype, bool full, int U, int mode, int shift) {
  if (dtype == QKNR_BF16)
    return U == 4 ? pick_seg<Bf16, 4>(full, U, mode, shift) : pick_seg<Bf16, 2>(full, U, mode, shift);
  return U == 4 ? pick_seg<Fp16, 4>(full, U, mode, shift) : pick_seg<Fp16, 2>(full, U, mode, shift);
}

const void* pick_elem_kernel(int dtype, int mode, int slots, int pw) {
  if (pw <= 2)
    return dtype == QKNR_BF16 ? pick_elem<Bf16, 3>(mode, slots, pw) : pick_elem<Fp16, 3>(mode, slots, pw);
  return dtype == QKNR_BF16 ? pick_elem<Bf16, 5>(mode, slots, pw) : pick_elem<Fp16, 5>(mode, slots, pw);
}

// NeoX pairs (d, d + R/2): with E elements per lane the partner sits a fixed
// m = (R/2)/E lanes away when R/2 is a multiple of E.
bool lanes_fit(int32_t R, int32_t neox, int E) {
  if (!neox) return true;
  return (R / 2) % E == 0 && R / 2 >= E;
}

// The fused op and the LayerNorm sibling also pair NeoX halves of 8m + 2,
// 8m + 4 and 8m + 6 dims on 16-byte lanes: each partner sits 2, 4 or 6 slots
// over in a neighbouring lane.
bool shifted_fits(int mode, int32_t R, int32_t neox) {
  const int s = (R / 2) % 8;
  return (mode == kFused || mode == kLayerRope) && neox && (s == 2 || s == 4 || s == 6);
}

// Partner slot shift of a lane mapping with E elements per lane: 0, or
// rope_dim/2 mod 8 where only the shifted pairing fits.
int lane_shift(int mode, int32_t R, int32_t neox, int E) {
  return (E == 8 && !lanes_fit(R, neox, 8) && shifted_fits(mode, R, neox)) ? (R / 2) % 8 : 0;
}

// Elements per lane of a run-time head_dim instance: 8 whenever the pairing
// allows it (shifted NeoX partners included, which covers every even NeoX
// half in the modes that take run-time head_dims). 0: none.
int any_dim_lanes(int mode, int32_t R, int32_t neox) {
  return (lanes_fit(R, neox, 8) || shifted_fits(mode, R, neox)) ? 8 : 0;
}

bool rotates(int mode) { return mode == kFused || mode == kRopeOnly || mode == kLayerRope; }

// The supported set (every mode, on the element-granular kernel): head_dim
// 2..512; with a rotation, rope_dim even in [2, head_dim].
bool elem_supported(int mode, int32_t D, int32_t R) {
  if (D < 2 || D > kElemMaxDim) return false;
  return !rotates(mode) || (R >= 2 && R <= D && R % 2 == 0);
}

// Shapes of the vectorised kernel in a mode: the page's rule (head_dim
// 64/128/256, rope_dim a multiple of head_dim/32, NeoX rotary lanes a power of
// two) widened to every even rope_dim for interleaved pairing, every NeoX
// rope_dim whose half is a multiple of some lane width (for the fused op: every
// even half), and other head_dims that are multiples of 8.
bool vector_shape(int mode, int32_t D, int32_t R, int32_t neox) {
  if (!fast_head_dim(D) && !any_head_dim(D)) return false;
  if (R <= 0 || R > D || R % 2) return false;
  if (!neox) return true;
  if (fast_head_dim(D)) {
    if (lanes_fit(R, neox, 8) || shifted_fits(mode, R, neox) || lanes_fit(R, neox, D / 32))
      return true;
    return D / 64 >= 2 && lanes_fit(R, neox, D / 64);
  }
  return any_dim_lanes(mode, R, neox) != 0;
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

// Vectorised instances exist for every mode at head_dim 64/128/256 and for the
// fused op and the LayerNorm sibling at the other multiples of 8.
bool vector_mode(int mode, int32_t D) {
  return fast_head_dim(D) ||
         (any_head_dim(D) && (mode == kFused || mode == kLayerRope || mode == kLayerOnly));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Launch defaults, chosen by measurement on MI355X (launch-shape sweeps over
// the benchmark workloads): one work item per wave with no persistent grid,
// 2 head groups per item, both loaded before the first is computed, 3 waves
// per workgroup when a head takes at most 16 lanes (head_dim <= 128 with
// 16-byte lanes; repeated A/Bs: +1.3-2% DiT, +0.4-3% Partial, GQA unchanged),
// 6 for the fused op at head_dim 256 with 16-byte lanes (32 lanes per head:
// +3.0% and +3.1% over 4 waves on two machines, 8 waves +2.4%, 5 waves +1.1%;
// the LayerNorm sibling there: 6 waves -0.5%, so it keeps 4) and 4 otherwise.
constexpr int kDefaultGroupsPerItem = 2;
constexpr int kDefaultUnroll = 2;
constexpr int kDefaultBlockWaves = 4;
constexpr int kDefaultBlockWavesNarrow = 3;  // lane groups of at most 16 lanes
constexpr int kDefaultBlockWavesHalf = 6;    // head_dim 256 on 16-byte lanes
// Run-time head_dim instances of the fused op and of the LayerNorm sibling take
// longer work items with NeoX pairing, or when a head group holds at most 640
// bytes (spare lanes in the padded lane group, or few heads per wave
// instruction): 4 head groups loaded together (unroll 4), 4 groups per item, 2
// waves per workgroup. At the same bytes per launch that measured faster on
// every run-time NeoX shape (fused op, head_dim 24-320: +2.5 to +33%, the most
// with 8-byte lanes) and on interleaved groups of at most 640 bytes (head_dim
// 40, 80, 144, 160, 320: +1 to +8%); the LayerNorm sibling gained 8-27% on the
// same shapes. Interleaved groups of 768-896 bytes lose 1.4-3.4% with it, and
// the compile-time head_dims 3.5-7.4% (4 groups per item at unroll 2), so they
// keep the usual defaults.
constexpr int kTailItems = 2048;  // shorter items at the end of a fused-op launch
constexpr int kLongItemGroupBytes = 640;
constexpr int kLongItemUnroll = 4;
constexpr int kLongItemGroups = 4;
constexpr int kLongItemBlockWaves = 2;
// element-granular kernel: heads per work item, in units of the heads it loads
// before computing the first (16 / slots)
constexpr int kDefaultElemRounds = 2;
// Element-granular instances that keep at most this many waves resident per
// SIMD (their register count decides it) are launched as a persistent grid
// (every wave loops over items) unless max_blocks is given: at the same bytes
// per launch that measured +4 to +20% on head_dim 40/38, 128/26, 72/70,
// 200/98, 66 NeoX and 130 interleaved (4 to 6 waves per SIMD; the LayerNorm
// sibling +10 to +26%), where a wave that ends leaves its slot idle while the
// next is launched and fetches its first loads. Instances holding 7 waves
// (head_dim 100, 50) lost 1-16% with it: their last round of items runs with
// part of the grid idle, which costs more than relaunches they already hide.
// Forced onto this kernel, head_dim 64-256 with either pairing (5 waves) gain
// 5-15% from it as well.
constexpr int kElemPersistentWaves = 6;
constexpr int kSimdsPerCu = 4;
// Work items per launch stay below 2^30 so a wave's item index plus the grid's
// wave count never overflows 32 bits.
constexpr int64_t kMaxItems = int64_t{1} << 30;

struct Plan {
  const void* fn = nullptr;
  int E = 8, L = 8, G = 8, ngq = 0, ng = 0, gpi = 0, nc = 0, U = kDefaultUnroll,
      wpb = kDefaultBlockWaves;
  int64_t items = 0;
  int max_blocks = 0;  // 0: one workgroup per wpb items; -1: occupancy x CUs; > 0: explicit cap
  int dmax = 0;        // head_dim of the instance (lane-group capacity)
  bool exact = true;   // head_dim == dmax
  bool elem = false;   // element-granular kernel (G = 1: a group is one head)
  int pw = 1;          // element-granular kernel: elements per lane slot (2-byte accesses x pw)
  bool seg = false;    // exact-fit lane groups of a run-time head_dim (L lanes, G heads)
  int shift = 0;       // NeoX partner slot shift (0, 2, 4 or 6)
  int64_t tail_item0 = -1;  // vectorised fused op: first item of the shorter last ones (-1: none)
  int64_t tail_t0 = 0;      // ... and its token
  int tail_nc = 1;          // such items per token (each holds gpi/2 groups)
  size_t lds = 0;      // dynamic LDS bytes per workgroup
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

// Plan of the vectorised kernel; the launch configuration's fields are
// already range-checked. QKNR_E_SHAPE: no lane mapping keeps the lane offsets
// of a head group below 2^31 (or too many work items).
int32_t make_plan(int mode, int64_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t R,
                  int32_t neox, int32_t dtype, int64_t q_head, int64_t k_head,
                  const qknr_launch_cfg& c, Plan* pl) {
  auto fits = [&](int E) {
    const int G = kWave / (D / E);
    return lane_offsets_fit(G, Hq, q_head, D) && lane_offsets_fit(G, Hkv, k_head, D);
  };
  int E = 0;
  bool seg = false;
  // head_dim 96 of the fused op (or the LayerNorm sibling) with a NeoX half
  // that is a multiple of 6 but not of 8: 12-byte lanes (16 lanes of 6
  // elements, no spare lanes) pair it at a whole-lane distance, where 16-byte
  // lanes would need shifted partners (measured 4-17% faster; with other
  // pairings the 16-byte lanes are 4% faster)
  const bool fit96 = D == 96 && (mode == kFused || mode == kLayerRope) && neox &&
                     lanes_fit(R, neox, 6) && (R / 2) % 8 != 0 &&
                     (c.lanes_per_head == 0 || c.lanes_per_head == 16);
  const bool exact = fast_head_dim(D) || fit96;
  const int dmax = exact ? D : any_dim_capacity(D);
  if (fit96) {
    E = 6;
    if (!fits(E)) return QKNR_E_SHAPE;
  } else if (!exact) {
    // run-time head_dim: 16-byte lanes in a lane group of dmax/8 lanes (every
    // even NeoX half pairs there, with shifted partners where needed)
    E = any_dim_lanes(mode, R, neox);
    if (E == 0) return QKNR_E_UNSUPPORTED;
    // NeoX partners 2 or 6 slots over (an LDS exchange per head group): heads
    // go into exact-fit lane groups of head_dim/8 lanes (up to 32) when that
    // fits at least 25% more heads into a wave instruction than the padded
    // groups (fused op: measured +2 to +18%; at fewer extra heads the tree
    // reduction it needs costs more than it saves), or 50% more for the
    // LayerNorm sibling, which reduces twice (+8 to +12% there; -8% at 25%)
    const int lanes = D / E, sh = lane_shift(mode, R, neox, E);
    const int g_pad = kWave / (dmax / E), g_fit = kWave / lanes;
    const bool more = mode == kFused ? 4 * g_fit >= 5 * g_pad
                                     : mode == kLayerRope && 2 * g_fit >= 3 * g_pad;
    // Partners 4 slots over (one ds_bpermute per element) gain from exact-fit
    // groups only in groups of 5 to 8 lanes (head_dim 40: +7.3% at rope_dim 40,
    // +8.8% at 24); head_dim 24 (3 lanes) lost 8.2% and groups of 9 or more
    // lanes 5-9% (the tree reduction and its broadcast cost more than the
    // busier lanes save)
    seg = ((sh == 2 || sh == 6) || (sh == 4 && mode == kFused && lanes >= 5 && lanes <= 8)) &&
          lanes <= 32 && more;
    const int G = kWave / (seg ? lanes : dmax / E);
    if (c.lanes_per_head != 0 && c.lanes_per_head != (seg ? lanes : dmax / E)) return QKNR_E_ARG;
    if (!lane_offsets_fit(G, Hq, q_head, D) || !lane_offsets_fit(G, Hkv, k_head, D))
      return QKNR_E_SHAPE;
  } else if (c.lanes_per_head == 0) {
    // 16-byte lanes first; then half a wave and a full wave per head
    const int cand[3] = {8, D / 32, D / 64};
    for (int e : cand) {
      const bool pairs = lanes_fit(R, neox, e) || (e == 8 && shifted_fits(mode, R, neox));
      if (e >= 2 && pairs && fits(e)) { E = e; break; }
    }
    if (E == 0) return QKNR_E_SHAPE;
  } else {
    if (c.lanes_per_head > kWave || D % c.lanes_per_head != 0) return QKNR_E_ARG;
    E = D / c.lanes_per_head;
    if (E != 8 && E != D / 32 && !(E == D / 64 && E >= 2)) return QKNR_E_ARG;
    if (!(lanes_fit(R, neox, E) || (E == 8 && shifted_fits(mode, R, neox))) || !fits(E))
      return QKNR_E_ARG;
  }
  const int L = seg ? D / E : dmax / E, G = kWave / L;
  const bool layer = mode == kLayerRope || mode == kLayerOnly;
  const bool long_items =
      (mode == kFused || layer) && !exact && (neox || G * 2 * D <= kLongItemGroupBytes);
  // the unfused baseline steps, and the LayerNorm sibling at head_dim
  // 64/128/256, exist at unroll 2; the run-time head_dims of the fused op and
  // the LayerNorm sibling at unroll 2 and 4 (1 runs as 2)
  int U = 2;
  if (mode == kFused && exact) U = c.unroll == 0 ? kDefaultUnroll : c.unroll;
  if ((mode == kFused || layer) && !exact && (c.unroll == 4 || (c.unroll == 0 && long_items)))
    U = kLongItemUnroll;
  // exact-fit groups of 5 lanes with NeoX partners 4 slots over (head_dim 40)
  // keep unroll 2 within their long items: 12 heads per wave instruction, 4
  // groups per item, +3.4 to +3.6% over unroll 4 at rope_dim 40, 24 and 8 (2
  // groups per item instead: -5.4%; head_dim 48 in groups of 6 lanes: -1.5%)
  if (seg && L == 5 && lane_shift(mode, R, neox, E) == 4 && c.unroll == 0) U = 2;

  pl->elem = false;
  pl->lds = 0;
  pl->shift = lane_shift(mode, R, neox, E);
  pl->E = E;
  pl->L = L;
  pl->dmax = dmax;
  pl->exact = exact;
  pl->G = G;
  pl->ngq = (Hq + pl->G - 1) / pl->G;
  pl->ng = pl->ngq + (Hkv + pl->G - 1) / pl->G;
  const int want_gpi = c.groups_per_item != 0 ? c.groups_per_item
                       : long_items          ? kLongItemGroups
                                             : kDefaultGroupsPerItem;
  pl->gpi = std::max(1, std::min(want_gpi, pl->ng));
  pl->nc = (pl->ng + pl->gpi - 1) / pl->gpi;
  pl->items = T * pl->nc;
  // The fused op on 16-byte lanes with its default items (several per token)
  // ends on about kTailItems items of half as many head groups: the last
  // waves of the launch are half as long, so the machine drains sooner
  // (one-group items after two-group ones: DiT +0.6%, GQA +0.6%, Partial
  // +0.3%, Large level; two-group items after the run-time head_dims' four:
  // +0.6 to +1.9% at head_dim 80 to 192). Not where a token is one or two
  // items (the 4+1-head GQA shard lost 5%), not with shifted NeoX partners
  // (head_dim 72: -1.2%), not in exact-fit groups and not on the 12-byte lanes
  // of head_dim 96.
  pl->tail_item0 = -1;
  pl->tail_t0 = 0;
  if (mode == kFused && E == 8 && !seg && pl->shift == 0 && c.groups_per_item == 0 &&
      (pl->gpi == 2 || pl->gpi == 4) && pl->nc >= 3) {
    const int tail_gpi = pl->gpi / 2;
    pl->tail_nc = (pl->ng + tail_gpi - 1) / tail_gpi;
    const int64_t tail = (kTailItems + pl->tail_nc - 1) / pl->tail_nc;  // tokens
    if (T >= 8 * tail) {
      pl->tail_t0 = T - tail;
      pl->tail_item0 = pl->tail_t0 * pl->nc;
      pl->items = pl->tail_item0 + tail * pl->tail_nc;
    }
  }
  if (pl->items > kMaxItems) return QKNR_E_SHAPE;
  pl->U = U;
  pl->wpb = c.block_waves != 0        ? c.block_waves
            : long_items              ? kLongItemBlockWaves
            : pl->L <= 16             ? kDefaultBlockWavesNarrow
            : mode == kFused && exact && pl->L == 32 && E == 8 ? kDefaultBlockWavesHalf
                                      : kDefaultBlockWaves;
  pl->max_blocks = c.max_blocks;
  // shifted partners: per wave, a row of 64 lanes x E floats (the exchange of
  // partners 2 or 6 slots over) followed by room for the token's cos|sin row
  // (up to 512 floats)
  if (pl->shift != 0)
    pl->lds = static_cast<size_t>(pl->wpb) * (kWave * E + 512) * sizeof(float);
  // NeoX instances at head_dim 64/128 on 16-byte lanes (the fused op and the
  // LayerNorm sibling): the token's cos|sin row per wave
  if (pl->shift == 0 && (mode == kFused || mode == kLayerRope) && exact && E == 8 && neox && D <= 128)
    pl->lds = static_cast<size_t>(pl->wpb) * D * sizeof(float);
  pl->seg = seg;
  pl->fn = seg ? pick_seg_kernel(dtype, R == D, U, mode, pl->shift)
               : pick_kernel(dtype, dmax, E, neox != 0, R == D, U, mode, exact, pl->shift);
  return pl->fn ? QKNR_OK : QKNR_E_UNSUPPORTED;
}

// Plan of the element-granular kernel. Runs of pw elements (accesses of 2*pw
// bytes): any pw in {8, 4, 2, 1} that divides head_dim and whose access size
// divides every pointer and used stride (align: their common alignment, 16 at
// most). A head takes L lanes of S runs each (L*S*pw >= head_dim, S*pw <= 8),
// a wave instruction G = 64/L heads of Q or of K of one token. Among the
// candidates (every allowed pw and S, with L rounded up to a power of two or
// exact), the plan takes the fewest wave instructions per token,
// S * (ceil(Hq/G) + ceil(Hkv/G)); ties go to a power-of-two L (DPP sums), then
// to the wider access, then to fewer slots. A group of several heads needs its
// lane offsets below 2^31; where they are not, one head per group is planned
// (its base address is 64-bit). 16/(S*pw) groups are loaded before the first is
// computed.
struct ElemShape {
  int pw = 1, S = 1, L = 64, G = 1;
  bool seg = false;
};

int pow2_at_least(int n) {
  int c = 1;
  while (c < n) c *= 2;
  return c;
}

ElemShape elem_shape(int32_t D, int align, int32_t Hq, int32_t Hkv, bool groups_fit) {
  ElemShape best;
  int64_t best_cost = INT64_MAX;
  auto consider = [&](int pw, int S, int L, bool seg) {
    const int G = groups_fit ? kWave / L : 1;
    const int64_t cost = static_cast<int64_t>(S) * ((Hq + G - 1) / G + (Hkv + G - 1) / G);
    // lexicographic: cost, then power-of-two lanes, then wider runs, then fewer slots
    const bool better = cost < best_cost ||
                        (cost == best_cost && (best.seg && !seg)) ||
                        (cost == best_cost && best.seg == seg && pw > best.pw) ||
                        (cost == best_cost && best.seg == seg && pw == best.pw && S < best.S);
    if (better) {
      best_cost = cost;
      best.pw = pw;
      best.S = S;
      best.L = L;
      best.G = G;
      best.seg = seg;
    }
  };
  for (int pw : {8, 4, 2, 1}) {
    if (D % pw != 0 || align < 2 * pw) continue;
    for (int S = 1; S * pw <= kElemPerLane; ++S) {
      const int lx = (D + S * pw - 1) / (S * pw);  // lanes a head needs
      if (lx > kWave) continue;
      const int lp = pow2_at_least(lx);
      consider(pw, S, lp, false);
      if (lx != lp && groups_fit) consider(pw, S, lx, true);
    }
  }
  return best;
}

int32_t make_elem_plan(int mode, int64_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t neox,
                       int32_t dtype, int align, int64_t q_head, int64_t k_head,
                       const qknr_launch_cfg& c, Plan* pl) {
  // several heads per group only where every group's lane offsets fit 32 bits
  const bool groups_fit = lane_offsets_fit(kWave, Hq, q_head, D) && lane_offsets_fit(kWave, Hkv, k_head, D);
  const ElemShape sh = elem_shape(D, align, Hq, Hkv, groups_fit);
  pl->elem = true;
  pl->shift = 0;
  pl->pw = sh.pw;
  pl->E = sh.S * sh.pw;
  pl->L = sh.L;
  pl->G = sh.G;
  pl->seg = sh.seg;
  pl->dmax = D;
  pl->exact = false;
  pl->ngq = (Hq + sh.G - 1) / sh.G;
  pl->ng = pl->ngq + (Hkv + sh.G - 1) / sh.G;
  const int U = 2 * kElemPerLane / pl->E;
  const int want = c.groups_per_item == 0 ? kDefaultElemRounds * U : c.groups_per_item;
  pl->gpi = std::max(1, std::min(want, pl->ng));
  pl->nc = (pl->ng + pl->gpi - 1) / pl->gpi;
  pl->items = T * pl->nc;
  if (pl->items > kMaxItems) return QKNR_E_SHAPE;
  pl->U = U;
  pl->wpb = c.block_waves == 0 ? kDefaultBlockWaves : c.block_waves;
  pl->max_blocks = c.max_blocks;
  // per wave: a row of 64 lanes x E floats (partners through LDS: NeoX, or
  // interleaved with single-element runs) and, with a rotation, room for one
  // cos|sin row plus a pad holding -0.0f and a discard area (the kernel's
  // layout; the exchange row is reserved in every instance)
  // (the LayerNorm sibling's 16-byte instances add a cos / sin pair per element
  // of a head: 2 * head_dim floats rounded up to 4)
  const int pairs = mode == kLayerRope && sh.pw == 8 ? (2 * D + 3) & ~3 : 0;
  pl->lds = static_cast<size_t>(pl->wpb) *
            (kWave * pl->E + (rotates(mode) ? kElemMaxDim + kElemRowPad : 0) + pairs) * sizeof(float);
  pl->fn = pick_elem_kernel(dtype, mode, sh.S, sh.pw);
  return pl->fn ? QKNR_OK : QKNR_E_UNSUPPORTED;
}

// Per-device CU count and per-kernel occupancy, computed once.
std::mutex g_cache_mu;
std::map<int, int> g_cus;
std::map<std::tuple<const void*, int, size_t>, int> g_occ;

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
  auto key = std::make_tuple(fn, threads, lds);
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

// q or k side of a call: base, weight and bias rows and the strides that are
// used (the token stride only with T > 1, the head stride only with H > 1)
// are multiples of `a` bytes.
bool side_aligned(const void* x, const void* w, const void* b, int64_t T, int32_t H, int64_t tok,
                  int64_t head, bool need_w, bool bias, uintptr_t a) {
  if (H == 0) return true;
  if (!aligned(x, a) || (need_w && !aligned(w, a)) || (bias && !aligned(b, a))) return false;
  return (T <= 1 || tok % static_cast<int64_t>(a) == 0) && (H <= 1 || head % static_cast<int64_t>(a) == 0);
}

// Validation (no HIP call) and planning. For kNormOnly the rotation arguments
// are ignored (pass rope_dim = head_dim); for kRopeOnly the weights and eps.
// The vectorised kernel is taken when the shape, the alignment and the lane
// offsets allow it (and the launch configuration does not ask for the
// element-granular kernel); every other supported case runs element-granular.
int32_t prepare(int mode, const Call& c, const qknr_launch_cfg* cfg, Plan* pl,
                qknr_launch_info* info) {
  if (c.T < 0 || c.Hq < 0 || c.Hkv < 0) return QKNR_E_SHAPE;
  if (c.dtype != QKNR_BF16 && c.dtype != QKNR_FP16) return QKNR_E_DTYPE;
  if (c.pdt != QKNR_I32 && c.pdt != QKNR_I64) return QKNR_E_DTYPE;
  if (!elem_supported(mode, c.D, c.R)) return QKNR_E_UNSUPPORTED;
  if (!std::isfinite(c.eps) || c.eps < 0.0f) return QKNR_E_ARG;
  if (c.T > INT32_MAX || c.T * (static_cast<int64_t>(c.Hq) + c.Hkv) > INT32_MAX) return QKNR_E_SHAPE;
  const qknr_launch_cfg lc = cfg ? *cfg : qknr_launch_cfg{0, 0, 0, 0, 0, 0};
  if (lc.lanes_per_head < 0 || lc.groups_per_item < 0 || lc.max_blocks < -1 ||
      lc.block_waves < 0 || lc.block_waves > kMaxBlockWaves ||
      (lc.unroll != 0 && lc.unroll != 1 && lc.unroll != 2 && lc.unroll != 4) ||
      (lc.generic != 0 && lc.generic != 1) || (lc.generic && lc.lanes_per_head))
    return QKNR_E_ARG;

  const bool empty = c.T == 0 || c.Hq + c.Hkv == 0;
  const bool need_w = mode != kRopeOnly;
  const bool need_rot = rotates(mode);
  const bool bias = (mode == kLayerRope || mode == kLayerOnly) && (c.bq || c.bk);
  bool vec_aligned = true;
  int elem_align = 16;  // common alignment of the views (2 to 16 bytes) for the element-granular kernel
  if (!empty) {
    if ((c.Hq > 0 && (!c.q || (need_w && !c.wq) || (bias && !c.bq))) ||
        (c.Hkv > 0 && (!c.k || (need_w && !c.wk) || (bias && !c.bk))) ||
        (need_rot && (!c.cache || !c.pos)))
      return QKNR_E_NULL;
    const int64_t vec = 2 * static_cast<int64_t>(c.D);
    if (c.Hq > 0 && !views_ok(c.T, c.Hq, c.qt, c.qh, vec)) return QKNR_E_SHAPE;
    if (c.Hkv > 0 && !views_ok(c.T, c.Hkv, c.kt, c.kh, vec)) return QKNR_E_SHAPE;
    if (!side_aligned(c.q, c.wq, c.bq, c.T, c.Hq, c.qt, c.qh, need_w, bias, 2) ||
        !side_aligned(c.k, c.wk, c.bk, c.T, c.Hkv, c.kt, c.kh, need_w, bias, 2))
      return QKNR_E_ALIGN;
    if (need_rot && (!aligned(c.cache, 4) || !aligned(c.pos, c.pdt == QKNR_I64 ? 8 : 4)))
      return QKNR_E_ALIGN;
    vec_aligned = side_aligned(c.q, c.wq, c.bq, c.T, c.Hq, c.qt, c.qh, need_w, bias, 16) &&
                  side_aligned(c.k, c.wk, c.bk, c.T, c.Hkv, c.kt, c.kh, need_w, bias, 16);
    while (elem_align > 2 &&
           !(side_aligned(c.q, c.wq, c.bq, c.T, c.Hq, c.qt, c.qh, need_w, bias, elem_align) &&
             side_aligned(c.k, c.wk, c.bk, c.T, c.Hkv, c.kt, c.kh, need_w, bias, elem_align)))
      elem_align /= 2;
  }

  const bool vector = !lc.generic && vec_aligned && vector_mode(mode, c.D) &&
                      vector_shape(mode, c.D, c.R, c.neox);
  int32_t rc = QKNR_E_UNSUPPORTED;
  if (vector) {
    rc = make_plan(mode, c.T, c.Hq, c.Hkv, c.D, c.R, c.neox, c.dtype, c.qh, c.kh, lc, pl);
    // an explicit lane mapping is honoured or refused, never replaced
    if (rc != QKNR_OK && (lc.lanes_per_head != 0 || rc != QKNR_E_SHAPE)) return rc;
  } else if (lc.lanes_per_head != 0) {
    return QKNR_E_ARG;
  }
  if (rc != QKNR_OK) {
    rc = make_elem_plan(mode, c.T, c.Hq, c.Hkv, c.D, c.neox, c.dtype, elem_align, c.qh, c.kh, lc, pl);
    if (rc != QKNR_OK) return rc;
  }
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
    info->generic = pl->elem ? 1 : 0;
    info->access_bytes = 2 * (pl->elem ? pl->pw : pl->E);
  }
  return QKNR_OK;
}

// Enqueue a prepared call (HIP calls from here on).
int32_t launch(const Call& c, const Plan& pl, qknr_launch_info* info) {
  if (c.T == 0 || c.Hq + c.Hkv == 0) return QKNR_OK;
  const int threads = pl.wpb * kWave;
  int cus = 0, per_cu = 0;
  const int32_t drc = device_limits(pl.fn, threads, pl.lds, &cus, &per_cu);
  if (drc != QKNR_OK) return drc;
  const int64_t needed = (pl.items + pl.wpb - 1) / pl.wpb;
  int64_t cap = needed;
  if (pl.max_blocks > 0) cap = pl.max_blocks;
  if (pl.max_blocks == -1 ||
      (pl.elem && pl.max_blocks == 0 && per_cu * pl.wpb <= kElemPersistentWaves * kSimdsPerCu))
    cap = static_cast<int64_t>(cus) * per_cu;
  const int grid = static_cast<int>(std::max<int64_t>(1, std::min(needed, cap)));
  if (info) info->grid_blocks = grid;

  char* qarg = static_cast<char*>(c.q);
  char* karg = static_cast<char*>(c.k);
  const void* wqarg = c.wq ? c.wq : c.wk;  // the side with 0 heads still gets a readable row
  const void* wkarg = c.wk ? c.wk : c.wq;
  const float* carg = c.cache;
  const void* parg = c.pos;
  const void* bqarg = c.bq ? c.bq : c.bk;  // the side with 0 heads still gets a readable row
  const void* bkarg = c.bk ? c.bk : c.bq;
  // head strides only matter for views with more than one head
  const int64_t qh = c.Hq > 1 ? c.qh : 0, kh = c.Hkv > 1 ? c.kh : 0;

  if (pl.elem) {
    ElemParams ep;
    ep.q_tok = c.qt;
    ep.k_tok = c.kt;
    ep.q_grp = qh * pl.G;
    ep.k_grp = kh * pl.G;
    // with one head per group only the 64-bit group stride is used
    ep.q_head = pl.G > 1 ? static_cast<uint32_t>(qh) : 0u;
    ep.k_head = pl.G > 1 ? static_cast<uint32_t>(kh) : 0u;
    ep.Hq = c.Hq;
    ep.Hkv = c.Hkv;
    ep.ngq = pl.ngq;
    ep.ng = pl.ng;
    ep.D = c.D;
    ep.R = c.R;
    ep.inv_d = static_cast<float>(1.0 / c.D);
    ep.eps = c.eps;
    ep.neox = c.neox ? 1 : 0;
    ep.pos64 = c.pdt == QKNR_I64;
    ep.has_bias = (c.bq || c.bk) ? 1 : 0;
    ep.cs2 = (reinterpret_cast<uintptr_t>(c.cache) % 8) == 0 ? 1 : 0;
    ep.L = pl.L;
    ep.G = pl.G;
    ep.seg = pl.seg ? 1 : 0;
    ep.gpi = pl.gpi;
    ep.nc = pl.nc;
    ep.n_items = static_cast<int32_t>(pl.items);
    void* args[] = {&qarg, &karg, &wqarg, &wkarg, &carg, &parg, &bqarg, &bkarg, &ep};
    if (hipLaunchKernel(pl.fn, dim3(grid), dim3(threads), args, pl.lds, c.stream) != hipSuccess)
      return QKNR_E_LAUNCH;
    return QKNR_OK;
  }

  Params prm;
  prm.has_bias = (c.bq || c.bk) ? 1 : 0;
  prm.cs_vec = (reinterpret_cast<uintptr_t>(c.cache) % 16 == 0) && ((c.R / 2) % 4 == 0);
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
  if (pl.seg) {
    prm.aux0 = pl.L;
    prm.aux1 = pl.G;
  } else {
    prm.aux0 = static_cast<int32_t>(pl.tail_item0 < 0 ? pl.items : pl.tail_item0);
    prm.aux1 = static_cast<int32_t>(pl.tail_t0);
  }
  void* args[] = {&qarg, &karg, &wqarg, &wkarg, &carg, &parg, &bqarg, &bkarg, &prm};
  if (hipLaunchKernel(pl.fn, dim3(grid), dim3(threads), args, pl.lds, c.stream) != hipSuccess)
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
  (void)is_neox;  // both pairings, every supported width
  return elem_supported(kFused, head_dim, rope_dim) ? 1 : 0;
}

QKNR_API const char* qknr_status_string(int32_t status) {
  switch (status) {
    case QKNR_OK: return "ok";
    case QKNR_E_NULL: return "qknr: a required pointer is NULL";
    case QKNR_E_SHAPE: return "qknr: bad shape or strides (negative, overlapping head vectors, or too large)";
    case QKNR_E_UNSUPPORTED:
      return "qknr: unsupported (head_dim, rope_dim): need head_dim in [2, 512] and, with a "
             "rotation, rope_dim even in [2, head_dim]";
    case QKNR_E_ALIGN:
      return "qknr: misaligned: q, k, weights, biases and q/k strides need 2-byte alignment, the "
             "cache 4 bytes, positions their element size";
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

QKNR_API int32_t qknr_layernorm_rope_inplace_ex(
    void* q, void* k, const void* wq, const void* wk, const void* bq, const void* bk,
    const float* cos_sin_cache, const void* positions, int64_t T, int32_t Hq, int32_t Hkv,
    int32_t head_dim, int32_t rope_dim, int32_t is_neox, float eps, int64_t q_tok_stride_B,
    int64_t q_head_stride_B, int64_t k_tok_stride_B, int64_t k_head_stride_B, int32_t dtype,
    int32_t pos_dtype, hipStream_t stream, const qknr_launch_cfg* cfg, qknr_launch_info* info) {
  const bool rotate = rope_dim != 0;
  const Call c{q, k, wq, wk, rotate ? cos_sin_cache : nullptr, rotate ? positions : nullptr, bq, bk,
               T, Hq, Hkv, head_dim, rotate ? rope_dim : head_dim, rotate ? is_neox : 0, eps,
               q_tok_stride_B, q_head_stride_B, k_tok_stride_B, k_head_stride_B, dtype,
               rotate ? pos_dtype : QKNR_I32, stream};
  Plan pl;
  const int32_t rc = prepare(rotate ? kLayerRope : kLayerOnly, c, cfg, &pl, info);
  return rc != QKNR_OK ? rc : launch(c, pl, info);
}

QKNR_API int32_t qknr_layernorm_rope_inplace(void* q, void* k, const void* wq, const void* wk,
                                             const void* bq, const void* bk,
                                             const float* cos_sin_cache, const void* positions,
                                             int64_t T, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                             int32_t rope_dim, int32_t is_neox, float eps,
                                             int64_t q_tok_stride_B, int64_t q_head_stride_B,
                                             int64_t k_tok_stride_B, int64_t k_head_stride_B,
                                             int32_t dtype, int32_t pos_dtype, hipStream_t stream) {
  return qknr_layernorm_rope_inplace_ex(q, k, wq, wk, bq, bk, cos_sin_cache, positions, T, Hq, Hkv,
                                        head_dim, rope_dim, is_neox, eps, q_tok_stride_B,
                                        q_head_stride_B, k_tok_stride_B, k_head_stride_B, dtype,
                                        pos_dtype, stream, nullptr, nullptr);
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
  char* d = static_cast<char*>(dst);
  const char* s = static_cast<const char*>(src);
  int64_t n = bytes / 16;
  void* args[] = {&d, &s, &n};
  return stream_launch(reinterpret_cast<const void*>(&copy_kernel), args, n, stream);
}

QKNR_API int32_t qknr_rmw(void* buf, int64_t bytes, uint32_t key, hipStream_t stream) {
  if (bytes < 0) return QKNR_E_SHAPE;
  if (bytes == 0) return QKNR_OK;
  if (!buf) return QKNR_E_NULL;
  if (!aligned(buf, 16) || bytes % 16) return QKNR_E_ALIGN;
  char* b = static_cast<char*>(buf);
  int64_t n = bytes / 16;
  void* args[] = {&b, &n, &key};
  return stream_launch(reinterpret_cast<const void*>(&rmw_kernel), args, n, stream);
}

}  // extern "C"
