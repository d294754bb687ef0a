/* Host-side validation driver for the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (device code untouched) and run
 * without a GPU.  It drives every entry point's argument checks, the
 * workspace size functions and the problem validator over a seeded sweep of
 * edge-valued shapes, dtypes, flags, pointers and strides.  No call here gets
 * as far as a kernel launch: every call either fails validation or is an
 * empty batch.  Exit status 0 = every invariant held; a sanitizer report
 * aborts the process with a non-zero status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_mi355x.h"

static int failures = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      if (failures < 20) {                                  \
        fprintf(stderr, "line %d: ", __LINE__);             \
        fprintf(stderr, __VA_ARGS__);                       \
        fprintf(stderr, "\n");                              \
      }                                                     \
      ++failures;                                           \
    }                                                       \
  } while (0)

/* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014) */
static uint64_t rng_state = 0x853c49e6748fea9bull;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
static int64_t pick(const int64_t* v, int n) { return v[next_u64() % (uint64_t)n]; }
#define PICK(arr) pick(arr, (int)(sizeof(arr) / sizeof(arr[0])))

static const int64_t Ts[] = {-1, 0, 1, 15, 16, 17, 32, 33, 255, 256, 257, 4096, 8192, 1 << 20, 1 << 28,
                             ((int64_t)1 << 31) - 1, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX, INT64_MIN};
static const int64_t Hs[] = {-8, 0, 1, 7, 8, 16, 128, 136, 256, 2560, 8192, 8200, 1 << 24, (1 << 24) + 8,
                             (int64_t)1 << 40, INT64_MAX};
static const int64_t Es[] = {-1, 0, 1, 2, 10, 16, 512, 1023, 1024, 1025, INT64_MAX};
static const int64_t ks[] = {-1, 0, 1, 2, 10, 63, 64, 65, 1024, INT64_MAX};
static const int64_t Is[] = {-8, 0, 1, 8, 72, 128, 640, 2048, 1 << 24, (1 << 24) + 8, INT64_MAX};
static const int64_t Iss[] = {-8, 0, 8, 40, 128, 640, 2048, 1 << 24, INT64_MAX};
static const int64_t dts[] = {-1, 0, 1, 2, 3, 1000};
static const int64_t sbs[] = {0, 64, 128, 256, -128};
static const int64_t ranks[] = {-16, 0, 8, 16, 17, 320, 65536, 65552, INT64_MAX};
static const int64_t slices[] = {-1, 0, 1, 2, 512, 65535, 65536, INT64_MAX};

static _Alignas(256) unsigned char buf[4096];

/* shapes the kernels take, so that most draws pass validation and reach the
 * size functions and the pointer checks */
static const int64_t gTs[] = {0, 1, 12, 16, 17, 37, 300, 2048, 4096, 8192, 65536};
static const int64_t gHs[] = {128, 256, 2560, 8192};
static const int64_t gEs[] = {1, 12, 64, 512, 1024};
static const int64_t gks[] = {1, 2, 8, 10};
static const int64_t gIs[] = {128, 640, 2048};
static const int64_t gIss[] = {0, 128, 640, 2048};

/* one field: an edge value one time in eight, else a good one */
#define FIELD(edge, good) (next_u64() % 8 == 0 ? PICK(edge) : PICK(good))

static void random_problem(moe_problem* p) {
  memset(p, 0, sizeof(*p));
  p->T = FIELD(Ts, gTs);
  p->H = FIELD(Hs, gHs);
  p->E = FIELD(Es, gEs);
  p->k = FIELD(ks, gks);
  p->I = FIELD(Is, gIs);
  p->I_shared = FIELD(Iss, gIss);
  p->act_dtype = (int32_t)(next_u64() % 8 == 0 ? PICK(dts) : 1);
  p->w_dtype = (int32_t)(next_u64() % 8 == 0 ? PICK(dts) : 1 + (int32_t)(next_u64() % 2));
  if (next_u64() % 8 == 0) p->act_dtype = p->w_dtype = MOE_F32;
  p->scale_block = (int32_t)(next_u64() % 8 == 0 ? PICK(sbs) : 128);
  p->flags = (uint32_t)(next_u64() % 8 == 0 ? next_u64() : next_u64() & 0x1f);
}

static void misaligned_weights(moe_weights* w, int off) {
  memset(w, 0, sizeof(*w));
  w->w_router = buf + off;
  w->w_gate = buf + 16 + off;
  w->w_up = buf + 32 + off;
  w->w_down = buf + 48 + off;
  w->stride_gate = w->stride_up = w->stride_down = (int64_t)(next_u64() % 5) - 1;
  w->s_gate = (const float*)(buf + 64 + off);
  w->s_up = (const float*)(buf + 80 + off);
  w->s_down = (const float*)(buf + 96 + off);
  w->sh_gate = buf + 112 + off;
  w->sh_up = buf + 128 + off;
  w->sh_down = buf + 144 + off;
  w->sh_gate_w = buf + 160 + off;
}

/* Every entry point with all pointers NULL: an error, or OK for an empty batch. */
static void null_calls(const moe_problem* p) {
  const int empty = p->T == 0;
  moe_status st[9];
  st[0] = moe_route(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  st[1] = moe_dispatch(p, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  st[2] = moe_expert_ffn(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  st[3] = moe_expert_gate_up(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  st[4] = moe_expert_down(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  st[5] = moe_combine(p, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
  st[6] = moe_layer_forward(p, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  st[7] = moe_layer_forward_noalloc(p, NULL, NULL, NULL, NULL, NULL, NULL);
  st[8] = moe_gr_write(p, NULL, NULL, NULL, NULL, NULL);
  for (int i = 0; i < 9; ++i) {
    EXPECT(st[i] != MOE_ERR_HIP, "entry %d reached a launch with NULL pointers", i);
    if (st[i] == MOE_OK) EXPECT(empty, "entry %d accepted NULL pointers for T=%lld", i, (long long)p->T);
  }
}

/* Misaligned (non-NULL) pointers and no workspace: never OK unless empty. */
static void misaligned_calls(const moe_problem* p) {
  moe_weights w;
  const int off = 1 + (int)(next_u64() % 15);
  misaligned_weights(&w, off);
  void* x = buf + 512 + off;
  void* out = buf + 1024 + off;
  moe_status a = moe_layer_forward(p, &w, x, out, NULL, NULL, NULL, 0, NULL);
  EXPECT(a != MOE_OK || p->T == 0, "layer_forward accepted misaligned pointers");
  EXPECT(a != MOE_ERR_HIP, "layer_forward reached a launch");
  moe_status b = moe_expert_ffn(p, &w, x, (const int32_t*)(buf + 2048 + off), (const int32_t*)(buf + 2304 + off),
                                out, NULL, NULL, 0, NULL);
  EXPECT(b != MOE_OK || p->T == 0, "expert_ffn accepted misaligned pointers");
  EXPECT(b != MOE_ERR_HIP, "expert_ffn reached a launch");
}

int main(void) {
  for (int s = 0; s <= 7; ++s) EXPECT(moe_status_str((moe_status)s) != NULL, "status string %d", s);
  EXPECT(moe_abi_version() == MOE_ABI_VERSION, "abi version");
  EXPECT(moe_validate(NULL) == MOE_ERR_NULL, "validate(NULL)");
  EXPECT(moe_workspace_bytes(NULL) == 0, "workspace_bytes(NULL)");

  long valid = 0, empty = 0;
  for (int it = 0; it < 200000; ++it) {
    moe_problem p;
    random_problem(&p);
    const moe_status v = moe_validate(&p);
    const size_t wb = moe_workspace_bytes(&p);
    EXPECT(v == moe_validate(&p), "validate not deterministic");
    if (v != MOE_OK) {
      EXPECT(wb == 0, "workspace for an invalid problem");
      continue;
    }
    ++valid;
    empty += p.T == 0;
    EXPECT(wb > 0 && wb % 256 == 0, "workspace %zu for a valid problem", wb);
    /* a smaller batch never needs more workspace */
    moe_problem q = p;
    q.T = p.T / 2;
    EXPECT(moe_validate(&q) == MOE_OK && moe_workspace_bytes(&q) <= wb, "workspace not monotone in T");
    null_calls(&p);
    misaligned_calls(&p);
    for (int r = 0; r < 3; ++r) {
      const int64_t rank = PICK(ranks);
      const size_t gb = moe_gr_workspace_bytes(&p, rank);
      moe_gr_weights g;
      memset(&g, 0, sizeof(g));
      g.rank = rank;
      const moe_status gs = moe_gr_read(&p, &g, NULL, NULL, NULL, NULL, gb, NULL);
      EXPECT(gs != MOE_ERR_HIP, "gr_read reached a launch");
      EXPECT(gs != MOE_OK || p.T == 0, "gr_read accepted NULL pointers");
    }
  }
  EXPECT(valid > 1000 && empty > 10, "sweep hit %ld valid problems (%ld empty)", valid, empty);

  /* allocation-free entry point: problems beyond its scratch are refused
   * before any device call */
  moe_problem big;
  memset(&big, 0, sizeof(big));
  big.T = 4096; big.H = 2560; big.E = 512; big.k = 10; big.I = 640; big.I_shared = 640;
  big.act_dtype = MOE_BF16; big.w_dtype = MOE_BF16; big.scale_block = 128;
  EXPECT(moe_workspace_bytes(&big) > MOE_NOALLOC_SCRATCH_BYTES, "big problem fits the scratch");
  moe_weights w;
  memset(&w, 0, sizeof(w));
  w.w_router = w.w_gate = w.w_up = w.w_down = w.sh_gate = w.sh_up = w.sh_down = w.sh_gate_w = buf;
  EXPECT(moe_layer_forward_noalloc(&big, &w, buf, buf + 256, NULL, NULL, NULL) == MOE_ERR_WORKSPACE,
         "noalloc did not refuse an oversized problem");

  /* audit and probe argument checks */
  for (int i = 0; i < (int)(sizeof(slices) / sizeof(slices[0])); ++i) {
    const size_t ab = moe_audit_workspace_bytes(slices[i]);
    EXPECT((ab > 0) == (slices[i] >= 1 && slices[i] <= 65535), "audit workspace for %lld slices",
           (long long)slices[i]);
    moe_audit_stats stats;
    EXPECT(moe_weight_audit(buf + 1, MOE_BF16, slices[i], 16, 16, &stats, buf, ab, NULL) != MOE_OK,
           "audit accepted an odd weight pointer");
    EXPECT(moe_weight_audit(buf, MOE_F32, 1, 16, 16, &stats, buf, ab, NULL) == MOE_ERR_UNSUPPORTED, "audit dtype");
    EXPECT(moe_weight_audit(buf, MOE_BF16, 1, 16, 8, &stats, buf, ab, NULL) == MOE_ERR_SHAPE, "audit stride");
  }
  uint32_t sink = 0;
  EXPECT(moe_hbm_read_probe(NULL, 16, &sink, NULL) == MOE_ERR_NULL, "probe NULL");
  EXPECT(moe_hbm_read_probe(buf + 4, 16, &sink, NULL) == MOE_ERR_ALIGN, "probe alignment");
  EXPECT(moe_hbm_read_probe(buf, 17, &sink, NULL) == MOE_ERR_ALIGN, "probe size");
  EXPECT(moe_hbm_read_probe(buf, 0, &sink, NULL) == MOE_OK, "probe empty");

  printf("valid %ld empty %ld failures %d\n", valid, empty, failures);
  return failures ? 1 : 0;
}
