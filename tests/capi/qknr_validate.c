/*
 * Drives the host side of libqknr.so through its C ABI without a GPU: every
 * rejection path of the entry points (each must return its documented status
 * before any HIP call), empty work, qknr_can_use over a grid of shapes,
 * qknr_status_string for every code, and -- only when the HIP runtime reports
 * no device -- valid calls that run the planners up to the device query
 * (they must return QKNR_E_DEVICE and fill the launch report). Built together
 * with the library's host code under AddressSanitizer by tests/test_asan.py;
 * any invalid memory access in the host code aborts the run.
 *
 * The pointers below are never dereferenced: the library only checks them for
 * NULL and alignment before it would hand them to a kernel, which no call here
 * reaches (no device). Exit status 0 on success, 1 with a message otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qknr.h"

static int failures = 0;

#define EXPECT(call, want)                                                         \
  do {                                                                             \
    int32_t got_ = (call);                                                         \
    if (got_ != (want)) {                                                          \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, \
              #call, (int)got_, (int)(want));                                      \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

/* addresses with a given alignment, never dereferenced */
#define PTR(a) ((void*)(uintptr_t)(a))

typedef struct {
  void *q, *k;
  const void *wq, *wk, *bq, *bk;
  const float* cache;
  const void* pos;
  int64_t T;
  int32_t Hq, Hkv, D, R, neox;
  float eps;
  int64_t qt, qh, kt, kh;
  int32_t dtype, pdt;
} Call;

static Call base_call(void) {
  Call c;
  c.q = PTR(0x100000);
  c.k = PTR(0x200000);
  c.wq = PTR(0x300000);
  c.wk = PTR(0x300100);
  c.bq = NULL;
  c.bk = NULL;
  c.cache = (const float*)PTR(0x400000);
  c.pos = PTR(0x500000);
  c.T = 7;
  c.Hq = 4;
  c.Hkv = 2;
  c.D = 128;
  c.R = 128;
  c.neox = 1;
  c.eps = 1e-6f;
  c.qt = 4 * 256;
  c.qh = 256;
  c.kt = 2 * 256;
  c.kh = 256;
  c.dtype = QKNR_BF16;
  c.pdt = QKNR_I64;
  return c;
}

static int32_t fused(const Call* c) {
  return qknr_inplace(c->q, c->k, c->wq, c->wk, c->cache, c->pos, c->T, c->Hq, c->Hkv, c->D,
                      c->R, c->neox, c->eps, c->qt, c->qh, c->kt, c->kh, c->dtype, c->pdt, NULL);
}

static int32_t fused_ex(const Call* c, const qknr_launch_cfg* cfg, qknr_launch_info* info) {
  return qknr_inplace_ex(c->q, c->k, c->wq, c->wk, c->cache, c->pos, c->T, c->Hq, c->Hkv, c->D,
                         c->R, c->neox, c->eps, c->qt, c->qh, c->kt, c->kh, c->dtype, c->pdt,
                         NULL, cfg, info);
}

static int32_t layer_ex(const Call* c, const qknr_launch_cfg* cfg, qknr_launch_info* info) {
  return qknr_layernorm_rope_inplace_ex(c->q, c->k, c->wq, c->wk, c->bq, c->bk, c->cache, c->pos,
                                        c->T, c->Hq, c->Hkv, c->D, c->R, c->neox, c->eps, c->qt,
                                        c->qh, c->kt, c->kh, c->dtype, c->pdt, NULL, cfg, info);
}

static void rejections(void) {
  Call c;
  /* NULL pointers */
  c = base_call(); c.q = NULL; EXPECT(fused(&c), QKNR_E_NULL);
  c = base_call(); c.k = NULL; EXPECT(fused(&c), QKNR_E_NULL);
  c = base_call(); c.wq = NULL; EXPECT(fused(&c), QKNR_E_NULL);
  c = base_call(); c.wk = NULL; EXPECT(fused(&c), QKNR_E_NULL);
  c = base_call(); c.cache = NULL; EXPECT(fused(&c), QKNR_E_NULL);
  c = base_call(); c.pos = NULL; EXPECT(fused(&c), QKNR_E_NULL);
  /* sizes and strides */
  c = base_call(); c.T = -1; EXPECT(fused(&c), QKNR_E_SHAPE);
  c = base_call(); c.Hq = -1; EXPECT(fused(&c), QKNR_E_SHAPE);
  c = base_call(); c.qh = 128; EXPECT(fused(&c), QKNR_E_SHAPE);          /* heads overlap */
  c = base_call(); c.qt = 512; EXPECT(fused(&c), QKNR_E_SHAPE);          /* tokens overlap */
  c = base_call(); c.kh = -256; EXPECT(fused(&c), QKNR_E_SHAPE);
  c = base_call(); c.T = (int64_t)1 << 40; c.qt = (int64_t)1 << 12; c.kt = (int64_t)1 << 12;
  EXPECT(fused(&c), QKNR_E_SHAPE);                                       /* T * heads overflows */
  /* shapes outside the supported set */
  c = base_call(); c.D = 1; c.R = 0; EXPECT(fused(&c), QKNR_E_UNSUPPORTED);
  c = base_call(); c.D = 513; c.R = 2; EXPECT(fused(&c), QKNR_E_UNSUPPORTED);
  c = base_call(); c.R = 127; EXPECT(fused(&c), QKNR_E_UNSUPPORTED);
  c = base_call(); c.R = 130; EXPECT(fused(&c), QKNR_E_UNSUPPORTED);
  /* dtype codes */
  c = base_call(); c.dtype = 7; EXPECT(fused(&c), QKNR_E_DTYPE);
  c = base_call(); c.pdt = 3; EXPECT(fused(&c), QKNR_E_DTYPE);
  /* alignment */
  c = base_call(); c.q = PTR(0x100001); EXPECT(fused(&c), QKNR_E_ALIGN);
  c = base_call(); c.wk = PTR(0x300101); EXPECT(fused(&c), QKNR_E_ALIGN);
  c = base_call(); c.cache = (const float*)PTR(0x400002); EXPECT(fused(&c), QKNR_E_ALIGN);
  c = base_call(); c.pos = PTR(0x500004); EXPECT(fused(&c), QKNR_E_ALIGN);  /* i64 positions */
  c = base_call(); c.kt = 2 * 256 + 1; EXPECT(fused(&c), QKNR_E_ALIGN);
  /* eps */
  c = base_call(); c.eps = -1.0f; EXPECT(fused(&c), QKNR_E_ARG);
  /* launch configurations */
  {
    qknr_launch_cfg bad[6];
    memset(bad, 0, sizeof bad);
    bad[0].block_waves = 9;
    bad[1].unroll = 3;
    bad[2].generic = 2;
    bad[3].max_blocks = -2;
    bad[4].generic = 1; bad[4].lanes_per_head = 16;
    bad[5].groups_per_item = -1;
    for (int i = 0; i < 6; ++i) {
      c = base_call();
      EXPECT(fused_ex(&c, &bad[i], NULL), QKNR_E_ARG);
      EXPECT(layer_ex(&c, &bad[i], NULL), QKNR_E_ARG);
    }
  }
  /* the LayerNorm sibling: one bias row only */
  c = base_call(); c.bq = PTR(0x600000); c.bk = NULL; c.Hkv = 2;
  EXPECT(layer_ex(&c, NULL, NULL), QKNR_E_NULL);
  /* the unfused steps */
  c = base_call();
  EXPECT(qknr_rmsnorm_inplace(NULL, c.k, c.wq, c.wk, c.T, c.Hq, c.Hkv, c.D, c.eps, c.qt, c.qh,
                              c.kt, c.kh, c.dtype, NULL), QKNR_E_NULL);
  EXPECT(qknr_rope_inplace(c.q, c.k, c.cache, c.pos, c.T, c.Hq, c.Hkv, c.D, 129, c.neox, c.qt,
                           c.qh, c.kt, c.kh, c.dtype, c.pdt, NULL), QKNR_E_UNSUPPORTED);
  EXPECT(qknr_unfused_inplace(c.q, c.k, c.wq, c.wk, c.cache, c.pos, c.T, c.Hq, c.Hkv, c.D, c.R,
                              c.neox, NAN, c.qt, c.qh, c.kt, c.kh, c.dtype, c.pdt, NULL),
         QKNR_E_ARG);
}

static void empty_work(void) {
  Call c = base_call();
  c.T = 0; c.q = NULL; c.k = NULL;
  EXPECT(fused(&c), QKNR_OK);
  c = base_call();
  c.Hq = 0; c.Hkv = 0;
  qknr_launch_info info;
  memset(&info, 0x5a, sizeof info);
  EXPECT(fused_ex(&c, NULL, &info), QKNR_OK);
  if (info.grid_blocks != 0) {
    fprintf(stderr, "empty work: grid_blocks %d, expected 0\n", (int)info.grid_blocks);
    ++failures;
  }
}

static void can_use_and_strings(void) {
  int n = 0;
  for (int D = 0; D <= 520; D += 1)
    for (int R = 0; R <= D + 2; R += (D < 40 ? 1 : 7))
      for (int neox = 0; neox < 2; ++neox) n += qknr_can_use(D, R, neox, QKNR_BF16, QKNR_I32);
  if (n == 0) {
    fprintf(stderr, "qknr_can_use accepted nothing\n");
    ++failures;
  }
  EXPECT(qknr_can_use(128, 128, 1, 9, QKNR_I32), 0);
  EXPECT(qknr_can_use(128, 128, 1, QKNR_FP16, 9), 0);
  for (int s = -12; s <= 3; ++s) {
    const char* t = qknr_status_string(s);
    if (t == NULL || strlen(t) == 0) {
      fprintf(stderr, "qknr_status_string(%d) is empty\n", s);
      ++failures;
    }
  }
}

/* Valid calls on every planner path; without a device each must stop at the
 * device query (QKNR_E_DEVICE) with its launch report filled. */
static void planners_without_device(void) {
  static const int shapes[][3] = {  /* head_dim, rope_dim, NeoX */
      {128, 128, 0}, {128, 128, 1}, {64, 32, 1}, {256, 256, 0}, {96, 24, 1}, {80, 20, 1},
      {136, 136, 1}, {40, 40, 1}, {72, 72, 1}, {40, 38, 1}, {100, 100, 1}, {130, 130, 0},
      {66, 66, 1}, {3, 2, 1}, {512, 512, 0}, {2, 2, 0}};
  const int n = (int)(sizeof shapes / sizeof shapes[0]);
  for (int i = 0; i < n; ++i) {
    for (int generic = 0; generic < 2; ++generic) {
      Call c = base_call();
      c.D = shapes[i][0];
      c.R = shapes[i][1];
      c.neox = shapes[i][2];
      c.qh = 2 * c.D + 32;
      c.qt = c.qh * c.Hq;
      c.kh = 2 * c.D + 32;
      c.kt = c.kh * c.Hkv;
      c.T = 1000;
      qknr_launch_cfg cfg;
      memset(&cfg, 0, sizeof cfg);
      cfg.generic = generic;
      qknr_launch_info info;
      memset(&info, 0, sizeof info);
      EXPECT(fused_ex(&c, &cfg, &info), QKNR_E_DEVICE);
      if (info.items <= 0 || info.lanes_per_head <= 0) {
        fprintf(stderr, "shape %d/%d generic %d: empty launch report\n", c.D, c.R, generic);
        ++failures;
      }
      memset(&info, 0, sizeof info);
      c.bq = PTR(0x600000);
      c.bk = PTR(0x600400);
      EXPECT(layer_ex(&c, &cfg, &info), QKNR_E_DEVICE);
    }
  }
}

int main(void) {
  rejections();
  empty_work();
  can_use_and_strings();
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess || devices == 0) {
    planners_without_device();
  } else {
    printf("a device is present: the planner cases (fake pointers) are skipped\n");
  }
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("qknr_validate: all checks passed\n");
  return 0;
}
