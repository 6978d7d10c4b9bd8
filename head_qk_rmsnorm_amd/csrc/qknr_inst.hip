// qknr_inst.hip -- one instance group of the fused QK RMSNorm + RoPE kernel
// table (see qknr_device.h). Built once per (I/O type, group) with
// -DQKNR_INST_IO=Bf16|Fp16 -DQKNR_INST_GROUP=0..5, so the groups compile in
// parallel; the host library (qknr.hip) calls pick_group<IO, GROUP> (the
// vectorised kernel: group 0 the fused op at head_dim 64/128/256, group 1 the
// other modes there, groups 2 and 4 the run-time head_dims at unroll 2 and 4)
// and pick_elem<IO, GROUP> (groups 3 and 5, the element-granular kernel with
// 2- and 4-byte, and 8- and 16-byte accesses).

#include "qknr_device.h"

#ifndef QKNR_INST_IO
#error "build with -DQKNR_INST_IO=Bf16 or Fp16"
#endif
#ifndef QKNR_INST_GROUP
#error "build with -DQKNR_INST_GROUP=0, 1, 2, 3, 4 or 5"
#endif

namespace qknr_impl {

template <class IO, int D, int E, bool NEOX, bool FULL, int GROUP>
const void* pick_unroll(int U, int mode) {
  if constexpr (GROUP == 0) {
    if (mode != kFused) return nullptr;
    switch (U) {
      case 1: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 1, kFused, true>);
      case 2: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 2, kFused, true>);
      case 4: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, E, NEOX, FULL, 4, kFused, true>);
      default: return nullptr;
    }
  } else {
    // the unfused baseline steps and the LayerNorm sibling exist at unroll 2 only
    if (mode == kFused || U != 2) return nullptr;
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
}

template <class IO, int D, int E, int GROUP>
const void* pick_pairing(bool neox, bool full, int U, int mode) {
  if (neox) {
    return full ? pick_unroll<IO, D, E, true, true, GROUP>(U, mode)
                : pick_unroll<IO, D, E, true, false, GROUP>(U, mode);
  }
  return full ? pick_unroll<IO, D, E, false, true, GROUP>(U, mode)
              : pick_unroll<IO, D, E, false, false, GROUP>(U, mode);
}

// Elements per lane: 8 (16-byte lanes), head_dim/32 (half a wave per head) and
// head_dim/64 (a full wave per head; needs an even count, so not head_dim 64).
template <class IO, int D, int GROUP>
const void* pick_lanes(int E, bool neox, bool full, int U, int mode) {
  if (E == 8) return pick_pairing<IO, D, 8, GROUP>(neox, full, U, mode);
  if constexpr (D / 32 != 8) {
    if (E == D / 32) return pick_pairing<IO, D, D / 32, GROUP>(neox, full, U, mode);
  }
  if constexpr (D / 64 >= 2 && D / 64 != 8) {
    if (E == D / 64) return pick_pairing<IO, D, D / 64, GROUP>(neox, full, U, mode);
  }
  return nullptr;
}

// Run-time head_dim instances: the fused op and the LayerNorm sibling at
// unroll UU (2 or 4), 16-byte lanes in a lane group of DMAX/8 lanes. Every even
// NeoX half pairs on them (shifted partners, below, where no lane divides it),
// so there are no narrower lanes.
template <class IO, int DMAX, int MODE, int UU>
const void* pick_any_dim_mode(bool neox, bool full) {
  if (neox) {
    return full ? reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, true, true, UU, MODE, false>)
                : reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, true, false, UU, MODE, false>);
  }
  return full ? reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, false, true, UU, MODE, false>)
              : reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, false, false, UU, MODE, false>);
}

template <class IO, int DMAX, int UU>
const void* pick_any_dim_lanes(int E, bool neox, bool full, int mode) {
  if (E != 8) return nullptr;
  if (mode == kFused) return pick_any_dim_mode<IO, DMAX, kFused, UU>(neox, full);
  if (mode == kLayerRope) return pick_any_dim_mode<IO, DMAX, kLayerRope, UU>(neox, full);
  if (mode == kLayerOnly)
    return reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, false, true, UU, kLayerOnly, false>);
  return nullptr;
}

// NeoX instances whose partners sit S = 2, 4 or 6 slots over (16-byte
// lanes): head_dim 64/128/256 with a partial rotation (a full one has
// rope_dim/2 a multiple of 8), the fused op at unroll 1, 2 and 4 in group 0 and
// the LayerNorm sibling at unroll 2 in group 1; the run-time head_dims of both
// at unroll 2 in group 2 and 4 in group 4.
template <class IO, int D, int S>
const void* pick_shift_exact(int U) {
  switch (U) {
    case 1: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, 8, true, false, 1, kFused, true, S>);
    case 2: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, 8, true, false, 2, kFused, true, S>);
    case 4: return reinterpret_cast<const void*>(&qknr_kernel<IO, D, 8, true, false, 4, kFused, true, S>);
    default: return nullptr;
  }
}

template <class IO, int DMAX, int UU, int MODE, int S>
const void* pick_shift_any(bool full) {
  return full ? reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, true, true, UU, MODE, false, S>)
              : reinterpret_cast<const void*>(&qknr_kernel<IO, DMAX, 8, true, false, UU, MODE, false, S>);
}

template <class IO, int DMAX, int UU, int S>
const void* pick_shift_mode(bool full, int mode) {
  return mode == kFused ? pick_shift_any<IO, DMAX, UU, kFused, S>(full)
                        : pick_shift_any<IO, DMAX, UU, kLayerRope, S>(full);
}

template <class IO, int GROUP, int S>
const void* pick_shift_of(int D, bool full, int U, int mode) {
  if constexpr (GROUP == 0) {
    if (full || mode != kFused) return nullptr;
    switch (D) {
      case 64: return pick_shift_exact<IO, 64, S>(U);
      case 128: return pick_shift_exact<IO, 128, S>(U);
      case 256: return pick_shift_exact<IO, 256, S>(U);
      default: return nullptr;
    }
  } else if constexpr (GROUP == 1) {
    if (full || mode != kLayerRope || U != 2) return nullptr;
    switch (D) {
      case 64: return reinterpret_cast<const void*>(&qknr_kernel<IO, 64, 8, true, false, 2, kLayerRope, true, S>);
      case 128: return reinterpret_cast<const void*>(&qknr_kernel<IO, 128, 8, true, false, 2, kLayerRope, true, S>);
      case 256: return reinterpret_cast<const void*>(&qknr_kernel<IO, 256, 8, true, false, 2, kLayerRope, true, S>);
      default: return nullptr;
    }
  } else if constexpr (GROUP == 2 || GROUP == 4) {
    constexpr int UU = GROUP == 2 ? 2 : 4;
    if (U != UU) return nullptr;
    switch (D) {  // the lane-group capacity DMAX
      case 16: return pick_shift_mode<IO, 16, UU, S>(full, mode);
      case 32: return pick_shift_mode<IO, 32, UU, S>(full, mode);
      case 64: return pick_shift_mode<IO, 64, UU, S>(full, mode);
      case 128: return pick_shift_mode<IO, 128, UU, S>(full, mode);
      case 256: return pick_shift_mode<IO, 256, UU, S>(full, mode);
      case 512: return pick_shift_mode<IO, 512, UU, S>(full, mode);
      default: return nullptr;
    }
  }
  return nullptr;
}

template <class IO, int GROUP>
const void* pick_shift(int D, bool full, int U, int mode, int shift) {
  if (mode != kFused && mode != kLayerRope) return nullptr;
  switch (shift) {
    case 2: return pick_shift_of<IO, GROUP, 2>(D, full, U, mode);
    case 4: return pick_shift_of<IO, GROUP, 4>(D, full, U, mode);
    case 6: return pick_shift_of<IO, GROUP, 6>(D, full, U, mode);
    default: return nullptr;
  }
}

template <class IO, int GROUP>
const void* pick_group(int D, int E, bool neox, bool full, int U, int mode, int shift) {
  if (shift != 0) return (neox && E == 8) ? pick_shift<IO, GROUP>(D, full, U, mode, shift) : nullptr;
  if constexpr (GROUP == 2 || GROUP == 4) {
    constexpr int UU = GROUP == 2 ? 2 : 4;
    if (U != UU) return nullptr;
    switch (D) {  // D is the lane-group capacity DMAX here
      case 16: return pick_any_dim_lanes<IO, 16, UU>(E, neox, full, mode);
      case 32: return pick_any_dim_lanes<IO, 32, UU>(E, neox, full, mode);
      case 64: return pick_any_dim_lanes<IO, 64, UU>(E, neox, full, mode);
      case 128: return pick_any_dim_lanes<IO, 128, UU>(E, neox, full, mode);
      case 256: return pick_any_dim_lanes<IO, 256, UU>(E, neox, full, mode);
      case 512: return pick_any_dim_lanes<IO, 512, UU>(E, neox, full, mode);
      default: return nullptr;
    }
  } else {
    switch (D) {
      case 64: return pick_lanes<IO, 64, GROUP>(E, neox, full, U, mode);
      case 128: return pick_lanes<IO, 128, GROUP>(E, neox, full, U, mode);
      case 256: return pick_lanes<IO, 256, GROUP>(E, neox, full, U, mode);
      case 96:  // 12-byte lanes: the fused op, and the LayerNorm sibling (partial NeoX)
        if constexpr (GROUP == 0) {
          if (E == 6) return pick_pairing<IO, 96, 6, GROUP>(neox, full, U, mode);
        } else if constexpr (GROUP == 1) {
          if (E == 6 && neox && !full && mode == kLayerRope && U == 2)
            return reinterpret_cast<const void*>(&qknr_kernel<IO, 96, 6, true, false, 2, kLayerRope, true>);
        }
        return nullptr;
      default: return nullptr;
    }
  }
}

// Exact-fit lane groups (SEG) for NeoX partners 2 or 6 slots over (the fused
// op and the LayerNorm sibling) and 4 slots over (the fused op): lanes per
// head and heads per wave instruction are run-time values, so DMAX plays no
// part (fixed at 256).
template <class IO, int UU, bool FULL, int MODE>
const void* pick_seg_shift(int shift) {
  switch (shift) {
    case 2: return reinterpret_cast<const void*>(&qknr_kernel<IO, 256, 8, true, FULL, UU, MODE, false, 2, true>);
    case 4:  // the fused op only: partners 4 slots over in groups of at most 8 lanes
      if constexpr (MODE == kFused)
        return reinterpret_cast<const void*>(&qknr_kernel<IO, 256, 8, true, FULL, UU, MODE, false, 4, true>);
      return nullptr;
    case 6: return reinterpret_cast<const void*>(&qknr_kernel<IO, 256, 8, true, FULL, UU, MODE, false, 6, true>);
    default: return nullptr;
  }
}

template <class IO, int GROUP>
const void* pick_seg(bool full, int U, int mode, int shift) {
  if constexpr (GROUP == 2 || GROUP == 4) {
    constexpr int UU = GROUP == 2 ? 2 : 4;
    if (U != UU) return nullptr;
    if (mode == kFused)
      return full ? pick_seg_shift<IO, UU, true, kFused>(shift) : pick_seg_shift<IO, UU, false, kFused>(shift);
    if (mode == kLayerRope)
      return full ? pick_seg_shift<IO, UU, true, kLayerRope>(shift)
                  : pick_seg_shift<IO, UU, false, kLayerRope>(shift);
    return nullptr;
  } else {
    return nullptr;
  }
}

#if QKNR_INST_GROUP == 3 || QKNR_INST_GROUP == 5
template <class IO, int MODE, int PW>
const void* pick_elem_slots(int slots) {
  switch (slots) {
    case 1: return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 1, PW>);
    case 2:
      if constexpr (2 * PW <= kElemPerLane) return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 2, PW>);
      return nullptr;
    case 3:
      if constexpr (3 * PW <= kElemPerLane) return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 3, PW>);
      return nullptr;
    case 4:
      if constexpr (4 * PW <= kElemPerLane) return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 4, PW>);
      return nullptr;
    case 5:
      if constexpr (PW == 1) return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 5, 1>);
      return nullptr;
    case 6:
      if constexpr (PW == 1) return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 6, 1>);
      return nullptr;
    case 7:
      if constexpr (PW == 1) return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 7, 1>);
      return nullptr;
    case 8:
      if constexpr (PW == 1) return reinterpret_cast<const void*>(&qknr_elem_kernel<IO, MODE, 8, 1>);
      return nullptr;
    default: return nullptr;
  }
}

// group 3: runs of 1 or 2 elements; group 5: runs of 4 or 8
template <class IO, int MODE>
const void* pick_elem_pw(int slots, int pw) {
  if constexpr (QKNR_INST_GROUP == 3) {
    switch (pw) {
      case 1: return pick_elem_slots<IO, MODE, 1>(slots);
      case 2: return pick_elem_slots<IO, MODE, 2>(slots);
      default: return nullptr;
    }
  } else {
    switch (pw) {
      case 4: return pick_elem_slots<IO, MODE, 4>(slots);
      case 8: return pick_elem_slots<IO, MODE, 8>(slots);
      default: return nullptr;
    }
  }
}

template <class IO, int GROUP>
const void* pick_elem(int mode, int slots, int pw) {
  switch (mode) {
    case kFused: return pick_elem_pw<IO, kFused>(slots, pw);
    case kNormOnly: return pick_elem_pw<IO, kNormOnly>(slots, pw);
    case kRopeOnly: return pick_elem_pw<IO, kRopeOnly>(slots, pw);
    case kLayerRope: return pick_elem_pw<IO, kLayerRope>(slots, pw);
    case kLayerOnly: return pick_elem_pw<IO, kLayerOnly>(slots, pw);
    default: return nullptr;
  }
}

template const void* pick_elem<QKNR_INST_IO, QKNR_INST_GROUP>(int, int, int);
#else
template const void* pick_group<QKNR_INST_IO, QKNR_INST_GROUP>(int, int, bool, bool, int, int, int);
template const void* pick_seg<QKNR_INST_IO, QKNR_INST_GROUP>(bool, int, int, int);
#endif

}  // namespace qknr_impl
