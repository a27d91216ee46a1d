// Drives every entry point of the C ABI's host code (csrc/api.hip, built with
// g++ under AddressSanitizer and UBSan against stand-in launchers) through its
// argument validation: NULL and misaligned pointers, descriptors out of range
// in every field, sizes near the 32-bit limits, and a seeded random sweep of
// descriptors.  Exits non-zero on the first unexpected status; the
// sanitizers abort on any out-of-bounds access or undefined behaviour.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>

#include "launch.h"
#include "sparse_attn.h"

namespace sa {
extern int g_calls;
extern Shape g_shape;
extern SelectParams g_sel;
extern FwdParams g_fwd;
extern BwdParams g_bwd;
}  // namespace sa

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);      \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static sa_desc base_desc() {
  sa_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 1;
  d.heads_q = 24;
  d.heads_kv = 24;
  d.seq_len = 8192;
  d.head_dim = 128;
  d.block = 64;
  d.dtype = SA_DTYPE_BF16;
  d.select_mode = SA_SELECT_DENSITY;
  d.density = 0.15;
  d.causal = 0;
  d.approx = 1;
  return d;
}

// fake, never dereferenced device addresses
static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

static sa_status call_all(const sa_desc* d, void* p, int which) {
  float* f = static_cast<float*>(p);
  int32_t* i = static_cast<int32_t*>(p);
  switch (which) {
    case 0: return sparse_attn_block_pool(d, p, p, p, f, f, f, p, nullptr);
    case 1: return sparse_attn_select(d, f, f, i, i, nullptr);
    case 2: return sparse_attn_route(d, p, p, p, f, f, f, p, i, i, nullptr);
    case 3: return sparse_attn_fwd(d, p, p, p, f, f, p, i, i, p, nullptr);
    case 4: return sparse_attn_fwd_lse(d, p, p, p, f, f, p, i, i, p, f, nullptr);
    case 5: return sparse_attn_bwd(d, p, p, p, p, i, i, p, f, p, f, (uint32_t*)p, i, i, f, f, p, p, p, nullptr);
    case 6: return sparse_attn_check_lists(d, i, i, (uint32_t*)p, nullptr);
  }
  return SA_OK;
}

int main() {
  // status strings, including codes outside the enum
  for (int c = -3; c < 20; ++c) CHECK(sparse_attn_status_string((sa_status)c) != nullptr);
  CHECK(strcmp(sparse_attn_status_string((sa_status)99), "unknown status") == 0);
  CHECK(sparse_attn_abi_version() == SPARSE_ATTN_ABI_VERSION);

  sa_desc d = base_desc();
  sa_sizes z;
  CHECK(sparse_attn_buffer_sizes(&d, &z) == SA_OK);
  CHECK(z.blk_idx == (size_t)24 * 128 * 128 * 4);
  CHECK(sparse_attn_buffer_sizes(nullptr, &z) == SA_ERR_NULL);
  CHECK(sparse_attn_buffer_sizes(&d, nullptr) == SA_ERR_NULL);

  // every compute entry: NULL pointers, misaligned pointers, then a valid call
  for (int w = 0; w < 7; ++w) {
    CHECK(call_all(&d, nullptr, w) == SA_ERR_NULL);
    CHECK(call_all(nullptr, P(0x1000), w) == SA_ERR_NULL);
    CHECK(call_all(&d, P(0x1004), w) == SA_ERR_ALIGN);
    const int before = sa::g_calls;
    CHECK(call_all(&d, P(0x1000), w) == SA_OK);
    CHECK(sa::g_calls == before + 1);
    CHECK(sa::g_shape.M == 128 && sa::g_shape.Hq == 24 && sa::g_shape.D == 128);
  }
  // parameters handed to the launchers
  d.scale = 0.f;
  CHECK(sparse_attn_select(&d, (float*)P(0x1000), (float*)P(0x1000), (int32_t*)P(0x1000), (int32_t*)P(0x1000),
                           nullptr) == SA_OK);
  CHECK(fabsf(sa::g_sel.scale - 1.0f / sqrtf(128.f)) < 1e-7f);
  CHECK(sa::g_sel.mode == SA_SELECT_DENSITY && sa::g_sel.force_diag == 0);
  d.causal = 1;
  d.scale = 0.25f;
  CHECK(sparse_attn_select(&d, (float*)P(0x1000), (float*)P(0x1000), (int32_t*)P(0x1000), (int32_t*)P(0x1000),
                           nullptr) == SA_OK);
  CHECK(sa::g_sel.scale == 0.25f && sa::g_sel.force_diag == 1 && sa::g_sel.causal == 1);
  // the backward takes bf16 only
  d = base_desc();
  d.dtype = SA_DTYPE_F32;
  CHECK(call_all(&d, P(0x1000), 5) == SA_ERR_UNSUPPORTED);

  // each descriptor field out of range
  struct Bad {
    void (*set)(sa_desc&);
    sa_status want;
  } bad[] = {
      {[](sa_desc& x) { x.batch = 0; }, SA_ERR_SHAPE},
      {[](sa_desc& x) { x.heads_q = -1; }, SA_ERR_SHAPE},
      {[](sa_desc& x) { x.heads_kv = 0; }, SA_ERR_SHAPE},
      {[](sa_desc& x) { x.heads_kv = 7; }, SA_ERR_SHAPE},
      {[](sa_desc& x) { x.seq_len = 0; }, SA_ERR_SHAPE},
      {[](sa_desc& x) { x.seq_len = -5; }, SA_ERR_SHAPE},
      {[](sa_desc& x) { x.head_dim = 96; }, SA_ERR_UNSUPPORTED},
      {[](sa_desc& x) { x.block = 32; }, SA_ERR_UNSUPPORTED},
      {[](sa_desc& x) { x.seq_len = 2049 * 64; }, SA_ERR_UNSUPPORTED},
      {[](sa_desc& x) { x.seq_len = INT32_MAX; }, SA_ERR_UNSUPPORTED},
      {[](sa_desc& x) { x.batch = 3000; x.heads_q = x.heads_kv = 30; }, SA_ERR_UNSUPPORTED},
      {[](sa_desc& x) { x.dtype = 9; }, SA_ERR_DTYPE},
      {[](sa_desc& x) { x.select_mode = 2; }, SA_ERR_PARAM},
      {[](sa_desc& x) { x.density = 0.0; }, SA_ERR_PARAM},
      {[](sa_desc& x) { x.density = NAN; }, SA_ERR_PARAM},
      {[](sa_desc& x) { x.select_mode = SA_SELECT_ALPHA; x.alpha = 1.5; }, SA_ERR_PARAM},
      {[](sa_desc& x) { x.causal = 2; }, SA_ERR_PARAM},
      {[](sa_desc& x) { x.approx = -1; }, SA_ERR_PARAM},
      {[](sa_desc& x) { x.scale = INFINITY; }, SA_ERR_PARAM},
  };
  for (auto& b : bad) {
    sa_desc x = base_desc();
    b.set(x);
    CHECK(sparse_attn_buffer_sizes(&x, &z) == b.want);
    for (int w = 0; w < 7; ++w) CHECK(call_all(&x, P(0x1000), w) == b.want);
  }

  // seeded sweep: random descriptors through every entry point; the status
  // must be one of the defined codes and a valid descriptor must give sizes
  // consistent with its shape
  std::mt19937_64 rng(12345);
  auto pick = [&](std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); };
  for (int it = 0; it < 20000; ++it) {
    sa_desc x;
    x.batch = (int32_t)pick({-1, 0, 1, 2, 7, 65535, 70000, INT32_MAX});
    x.heads_q = (int32_t)pick({-8, 0, 1, 2, 8, 24, 32, 40, 65535, INT32_MAX});
    x.heads_kv = (int32_t)pick({-1, 0, 1, 2, 8, 24, 3});
    x.seq_len = (int32_t)pick({-1, 0, 1, 63, 64, 1000, 8192, 32760, 131072, 262144, 262145, INT32_MAX});
    x.head_dim = (int32_t)pick({0, 64, 96, 128, 256});
    x.block = (int32_t)pick({0, 64, 128, 100});
    x.dtype = (int32_t)pick({0, 1, 2});
    x.select_mode = (int32_t)pick({0, 1, 5});
    x.alpha = (double)pick({-1, 0, 1, 2}) * 0.5;
    x.density = (double)pick({-1, 0, 1, 2, 3}) * 0.4;
    x.scale = (float)pick({-1, 0, 1}) * 0.125f;
    x.causal = (int32_t)pick({0, 1, 3});
    x.approx = (int32_t)pick({0, 1, -2});
    const sa_status s = sparse_attn_buffer_sizes(&x, &z);
    CHECK(s >= SA_OK && s <= SA_ERR_HIP);
    if (s == SA_OK) {
      const size_t M = (size_t)(x.seq_len + x.block - 1) / x.block;
      CHECK(z.blk_cnt == (size_t)x.batch * x.heads_q * M * 4);
      CHECK(z.blk_idx == z.blk_cnt * M);
      sa_bwd_sizes bz;
      CHECK(sparse_attn_bwd_buffer_sizes(&x, &bz) == SA_OK);
    }
    for (int w = 0; w < 7; ++w) {
      const sa_status t = call_all(&x, P(0x2000), w);
      CHECK(t == s || (s == SA_OK && w == 5 && t == SA_ERR_UNSUPPORTED));
    }
  }
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("host validation: all checks passed (%d launches recorded)\n", sa::g_calls);
  return 0;
}
