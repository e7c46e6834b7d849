// Host-side paths of the C ABI, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code (device code is untouched): every entry point with invalid arguments (each must
// return its status before anything is enqueued), the workspace and plan queries over the
// workloads' shapes and extreme descriptor values, the table hooks and the trace objects. No
// kernel is launched and no device memory is touched, so this runs without a GPU. Exit status 0
// when every call returned what the ABI documents; a sanitizer report aborts the process.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "bd.h"

static int failures = 0;

static void expect(bd_status got, bd_status want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, bd_last_error());
    ++failures;
  } else if (want != BD_OK && std::strlen(bd_last_error()) == 0) {
    std::printf("FAIL %s: no error message\n", what);
    ++failures;
  }
}

static bd_attn_desc attn(int B, int Hq, int Hkv, int D, int S, int64_t L) {
  bd_attn_desc d;
  std::memset(&d, 0, sizeof(d));
  d.batch = B;
  d.n_q_heads = Hq;
  d.n_kv_heads = Hkv;
  d.head_dim = D;
  d.block_len = S;
  d.prefix_capacity = L;
  d.max_prefix_len = L;
  return d;
}

static bd_unmask_desc unmask(int B, int S, int V) {
  bd_unmask_desc d;
  std::memset(&d, 0, sizeof(d));
  d.batch = B;
  d.block_len = S;
  d.vocab = V;
  d.row_stride = V;
  d.logits_dtype = BD_BF16;
  d.gamma = 0.9f;
  d.min_commit = 1;
  return d;
}

int main() {
  // fake, aligned, never dereferenced device addresses: validation must stop before any use
  void* p = reinterpret_cast<void*>(uintptr_t(1) << 20);
  void* odd = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2);
  const int32_t* pl = static_cast<const int32_t*>(p);

  // ---- attention: descriptors
  expect(bd_attn_step(nullptr, p, p, p, p, p, pl, nullptr, p, nullptr, p, 1 << 20, nullptr), BD_EINVAL, "null desc");
  struct Case { bd_attn_desc d; bd_status want; const char* what; };
  std::vector<Case> bad;
  auto mk = [&](void (*f)(bd_attn_desc&), bd_status want, const char* what) {
    bd_attn_desc d = attn(2, 32, 2, 128, 16, 4096);
    f(d);
    bad.push_back({d, want, what});
  };
  mk([](bd_attn_desc& d) { d.batch = 0; }, BD_EINVAL, "batch 0");
  mk([](bd_attn_desc& d) { d.batch = -7; }, BD_EINVAL, "batch < 0");
  mk([](bd_attn_desc& d) { d.n_kv_heads = 3; }, BD_EINVAL, "Hq % Hkv");
  mk([](bd_attn_desc& d) { d.n_kv_heads = 0; }, BD_EINVAL, "Hkv 0");
  mk([](bd_attn_desc& d) { d.head_dim = 96; }, BD_EUNSUPPORTED, "head_dim 96");
  mk([](bd_attn_desc& d) { d.block_len = 65; }, BD_EINVAL, "S 65");
  mk([](bd_attn_desc& d) { d.prefix_capacity = 0; }, BD_EINVAL, "capacity 0");
  mk([](bd_attn_desc& d) { d.prefix_capacity = INT64_MAX; }, BD_EUNSUPPORTED, "capacity huge");
  mk([](bd_attn_desc& d) { d.max_prefix_len = 4097; }, BD_EINVAL, "max_prefix_len > capacity");
  mk([](bd_attn_desc& d) { d.max_prefix_len = -1; }, BD_EINVAL, "max_prefix_len < 0");
  mk([](bd_attn_desc& d) { d.softmax_scale = NAN; }, BD_EINVAL, "scale NaN");
  mk([](bd_attn_desc& d) { d.softmax_scale = INFINITY; }, BD_EINVAL, "scale inf");
  mk([](bd_attn_desc& d) { d.num_splits = -1; }, BD_EINVAL, "num_splits < 0");
  mk([](bd_attn_desc& d) { d.causal = 2; }, BD_EINVAL, "causal 2");
  mk([](bd_attn_desc& d) { d.n_q_heads = 1 << 30; d.n_kv_heads = 1; d.block_len = 64; }, BD_EUNSUPPORTED, "rows 2^36");
  for (auto& c : bad) {
    expect(bd_attn_step(&c.d, p, p, p, p, p, pl, nullptr, p, nullptr, p, 1 << 20, nullptr), c.want, c.what);
    if (bd_attn_workspace_bytes(&c.d) != 0) { std::printf("FAIL workspace of %s\n", c.what); ++failures; }
    bd_attn_plan_info info;
    expect(bd_attn_plan(&c.d, &info), c.want, c.what);
    expect(bd_kv_append(&c.d, p, p, p, p, static_cast<int32_t*>(p), nullptr, nullptr), c.want, c.what);
  }
  // ---- attention: pointers and workspace
  bd_attn_desc good = attn(2, 32, 2, 128, 16, 4096);
  const size_t nb = bd_attn_workspace_bytes(&good);
  if (nb == 0) { std::printf("FAIL split workspace 0\n"); ++failures; }
  for (int i = 0; i < 6; ++i) {
    void* a[6] = {p, p, p, p, p, p};
    a[i] = nullptr;
    expect(bd_attn_step(&good, a[0], a[1], a[2], a[3], a[4], static_cast<const int32_t*>(a[5]), nullptr, p, nullptr, p,
                        nb, nullptr), BD_EINVAL, "null input");
    a[i] = odd;
    expect(bd_attn_step(&good, a[0], a[1], a[2], a[3], a[4], static_cast<const int32_t*>(a[5]), nullptr, p, nullptr, p,
                        nb, nullptr), BD_EINVAL, "misaligned input");
  }
  expect(bd_attn_step(&good, p, p, p, p, p, pl, nullptr, nullptr, nullptr, p, nb, nullptr), BD_EINVAL, "null out");
  expect(bd_attn_step(&good, p, p, p, p, p, pl, nullptr, p, nullptr, p, nb - 1, nullptr), BD_EWORKSPACE, "small ws");
  expect(bd_attn_step(&good, p, p, p, p, p, pl, nullptr, p, nullptr, nullptr, nb, nullptr), BD_EINVAL, "null ws");
  expect(bd_attn_step(&good, p, p, p, p, p, pl, nullptr, p, nullptr, odd, nb, nullptr), BD_EINVAL, "misaligned ws");
  expect(bd_attn_plan(&good, nullptr), BD_EINVAL, "plan info NULL");
  bd_attn_desc full = attn(2, 32, 2, 128, 16, 4096);
  full.max_prefix_len = 4090;
  expect(bd_kv_append(&full, p, p, p, p, static_cast<int32_t*>(p), nullptr, nullptr), BD_EINVAL, "append past capacity");
  expect(bd_kv_append(&good, nullptr, p, p, p, static_cast<int32_t*>(p), nullptr, nullptr), BD_EINVAL, "append null");
  // ---- plans and workspace sizes over the workloads' shapes and large values (UBSan: overflows)
  const int64_t shapes[][6] = {{1, 8, 2, 64, 16, 256},      {1, 32, 2, 128, 16, 4096},   {32, 32, 2, 128, 16, 8192},
                               {32, 32, 2, 128, 32, 8192},  {4, 32, 2, 128, 16, 65536},  {1, 32, 2, 128, 16, 262144},
                               {16, 32, 8, 128, 16, 32768}, {4096, 64, 1, 128, 64, 8388607 / 128}, {1, 1, 1, 64, 1, 1},
                               {100000, 2, 2, 64, 1, 16}};
  for (auto& sh : shapes) {
    for (int ns : {0, 1, 7, 1000}) {
      bd_attn_desc d = attn((int)sh[0], (int)sh[1], (int)sh[2], (int)sh[3], (int)sh[4], sh[5]);
      d.num_splits = ns;
      bd_attn_plan_info info;
      const bd_status st = bd_attn_plan(&d, &info);
      if (st == BD_EUNSUPPORTED) {
        // the largest shapes with forced splits exceed one launch's grid: refused, with no workspace
        if (!std::strstr(bd_last_error(), "too large for one launch") || bd_attn_workspace_bytes(&d) != 0) {
          std::printf("FAIL oversize plan not reported as such\n");
          ++failures;
        }
        continue;
      }
      expect(st, BD_OK, "plan");
      if (info.workgroups < 1 || info.num_splits < 1 || info.chunk_keys < 64) { std::printf("FAIL plan values\n"); ++failures; }
      (void)bd_attn_workspace_bytes(&d);
      bd_unmask_desc u = unmask((int)sh[0], (int)sh[4], 131072);
      (void)bd_denoise_workspace_bytes(&d, &u);
    }
  }
  // ---- unmasking
  bd_unmask_desc ug = unmask(2, 16, 131072);
  const size_t ub = bd_unmask_workspace_bytes(&ug);
  expect(bd_confidence_unmask(nullptr, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL,
         "unmask null desc");
  {
    bd_unmask_desc u = ug; u.gamma = NAN;
    expect(bd_confidence_unmask(&u, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "gamma NaN");
    u = ug; u.row_stride = 100;
    expect(bd_confidence_unmask(&u, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "stride");
    u = ug; u.vocab = 1001; u.row_stride = 1001;
    expect(bd_confidence_unmask(&u, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "stride bytes");
    u = ug; u.logits_dtype = (bd_dtype)9;
    expect(bd_confidence_unmask(&u, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "dtype");
    u = ug; u.commit_all = 3;
    expect(bd_confidence_unmask(&u, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "flags");
  }
  expect(bd_confidence_unmask(&ug, nullptr, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "null logits");
  expect(bd_confidence_unmask(&ug, odd, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "odd logits");
  expect(bd_confidence_unmask(&ug, p, nullptr, (int32_t*)p, nullptr, nullptr, nullptr, p, ub, nullptr), BD_EINVAL, "null mask");
  expect(bd_confidence_unmask(&ug, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, p, ub - 1, nullptr), BD_EWORKSPACE, "small");
  {
    bd_unmask_desc big = unmask(5462, 64, 4096);
    big.logits_dtype = BD_F32;
    expect(bd_confidence_unmask_noalloc(&big, p, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, nullptr),
           BD_EUNSUPPORTED, "noalloc bound");
    expect(bd_confidence_unmask_noalloc(&ug, nullptr, (uint8_t*)p, (int32_t*)p, nullptr, nullptr, nullptr, nullptr),
           BD_EINVAL, "noalloc null logits");
  }
  expect(bd_spec_verify(&ug, p, nullptr, (const int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p, p, ub, nullptr),
         BD_EINVAL, "spec null draft");
  expect(bd_spec_verify(&ug, p, (const int32_t*)p, (const int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p, p, ub - 1,
                        nullptr), BD_EWORKSPACE, "spec small ws");
  // ---- halting
  {
    bd_halt_desc h;
    std::memset(&h, 0, sizeof(h));
    h.batch = 2; h.n_per_seq = 4096; h.dtype = BD_BF16; h.eps = 1e-3f; h.max_iter = 4;
    const size_t hb = bd_loop_halt_workspace_bytes(&h);
    expect(bd_loop_halt(&h, p, p, 0, nullptr, (uint8_t*)p, p, hb, nullptr), BD_EINVAL, "iteration 0");
    expect(bd_loop_halt(&h, p, nullptr, 1, nullptr, (uint8_t*)p, p, hb, nullptr), BD_EINVAL, "null state");
    expect(bd_loop_halt(&h, p, p, 1, nullptr, (uint8_t*)p, p, hb - 1, nullptr), BD_EWORKSPACE, "halt ws");
    bd_halt_desc h2 = h; h2.n_per_seq = 4097;
    expect(bd_loop_halt(&h2, p, p, 1, nullptr, (uint8_t*)p, p, 1 << 20, nullptr), BD_EINVAL, "halt row bytes");
    h2 = h; h2.eps = -1.f;
    expect(bd_loop_halt(&h2, p, p, 1, nullptr, (uint8_t*)p, p, 1 << 20, nullptr), BD_EINVAL, "eps < 0");
    h2 = h; h2.n_per_seq = INT64_MAX / 2;
    (void)bd_loop_halt_workspace_bytes(&h2);
  }
  // ---- the loop
  {
    bd_step_hooks hooks;
    std::memset(&hooks, 0, sizeof(hooks));
    bd_step_table tab;
    std::memset(&tab, 0, sizeof(tab));
    expect(bd_table_hooks(&tab, &hooks), BD_EINVAL, "empty table");
    const void* ptrs[2] = {p, p};
    tab.q = ptrs; tab.k_blk = ptrs; tab.v_blk = ptrs; tab.logits = ptrs; tab.n_steps = 2;
    expect(bd_table_hooks(&tab, &hooks), BD_OK, "table hooks");
    const size_t lb = bd_denoise_workspace_bytes(&good, &ug);
    int32_t* i32 = static_cast<int32_t*>(p);
    expect(bd_denoise_block(&good, &ug, 0, 0, &hooks, p, p, pl, p, (uint8_t*)p, i32, i32, nullptr, p, lb, nullptr),
           BD_EINVAL, "T 0");
    expect(bd_denoise_block(&good, &ug, 8, 8, &hooks, p, p, pl, p, (uint8_t*)p, i32, i32, nullptr, p, lb, nullptr),
           BD_EINVAL, "t0 >= T");
    expect(bd_denoise_block(&good, &ug, 8, 0, nullptr, p, p, pl, p, (uint8_t*)p, i32, i32, nullptr, p, lb, nullptr),
           BD_EINVAL, "no hooks");
    expect(bd_denoise_block(&good, &ug, 8, 0, &hooks, p, p, pl, p, (uint8_t*)p, i32, nullptr, nullptr, p, lb, nullptr),
           BD_EINVAL, "no steps_used");
    expect(bd_denoise_block(&good, &ug, 8, 0, &hooks, p, p, pl, p, (uint8_t*)p, i32, i32, nullptr, p, lb - 1, nullptr),
           BD_EWORKSPACE, "loop ws");
    bd_unmask_desc u32 = ug;
    u32.block_len = 32;
    expect(bd_denoise_block(&good, &u32, 8, 0, &hooks, p, p, pl, p, (uint8_t*)p, i32, i32, nullptr, p, lb, nullptr),
           BD_EINVAL, "descriptors disagree");
  }
  // ---- traces (no GPU needed for the invalid ones; a valid one may or may not find a device)
  {
    bd_trace* t = nullptr;
    expect(bd_trace_create(0, &t), BD_EINVAL, "trace capacity 0");
    expect(bd_trace_create(4, nullptr), BD_EINVAL, "trace out NULL");
    if (bd_trace_count(nullptr) != 0) { std::printf("FAIL trace count NULL\n"); ++failures; }
    expect(bd_trace_get(nullptr, 0, nullptr, nullptr), BD_EINVAL, "trace get NULL");
    expect(bd_trace_clear(nullptr), BD_EINVAL, "trace clear NULL");
    bd_trace_destroy(nullptr);
    bd_status st = bd_trace_create(8, &t);
    if (st == BD_OK) {
      expect(bd_trace_get(t, 0, nullptr, nullptr), BD_EINVAL, "trace get empty");
      expect(bd_trace_attach(t), BD_OK, "attach");
      expect(bd_trace_attach(nullptr), BD_OK, "detach");
      bd_trace_destroy(t);
    } else if (st != BD_EHIP) {
      std::printf("FAIL trace create status %d\n", (int)st);
      ++failures;
    }
  }
  if (std::strstr(bd_version(), "gfx950") == nullptr) { std::printf("FAIL version\n"); ++failures; }
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
