// Host-side check of the library's descriptor validation and size queries,
// built together with the library's host code under AddressSanitizer and
// UndefinedBehaviorSanitizer (no device code, no GPU). Every descriptor is
// passed through validate and the size queries of the layer, the stack and
// the LM head; entry points are called only with arguments that must be
// refused before any launch (NULL or misaligned pointers, short workspaces),
// and the test fails if one of them is not. Signed overflow in the size
// arithmetic, out-of-bounds accesses and use of uninitialised plan fields are
// reported by the sanitizers and end the run with a non-zero status.
#include "bpt.h"

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
template <typename T, size_t N>
T pick(const T (&v)[N]) { return v[next_u64() % N]; }

int failures = 0;
void expect(bool ok, const char* what, const char* detail) {
  if (!ok) {
    ++failures;
    std::printf("FAIL %s: %s\n", what, detail);
  }
}

bpt_layer_desc base_desc() {
  bpt_layer_desc d;
  std::memset(&d, 0, sizeof d);
  d.abi_version = BPT_ABI_VERSION;
  d.dtype = BPT_BF16;
  d.norm = BPT_LAYERNORM;
  d.ffn = BPT_GELU_ERF;
  d.causal = 1;
  d.batch = 1;
  d.seq_len = 4096;
  d.hidden = 2048;
  d.n_heads = 16;
  d.n_kv_heads = 16;
  d.head_dim = 128;
  d.ffn_dim = 8192;
  d.q_block = 512;
  d.kv_block = 512;
  d.head_chunk = 16;
  d.rope_base = 10000.0;
  d.norm_eps = 1e-5f;
  d.window = 0;
  d.dropout_p = 0.f;
  d.seed = 0;
  return d;
}

// Interesting values per field: valid ones, boundaries and hostile ones.
const int64_t kI64[] = {0, 1, -1, 2, 3, 8, 16, 32, 63, 64, 96, 128, 256, 512, 784, 1000, 1024,
                        2048, 4096, 8192, 16384, 32768, 65536, 131072, 1 << 20, 1LL << 31,
                        (1LL << 31) - 1, 1LL << 40, std::numeric_limits<int64_t>::max(),
                        std::numeric_limits<int64_t>::min()};
const int32_t kI32[] = {0, 1, 2, 3, -1, 7, 100, 4096, std::numeric_limits<int32_t>::max(),
                        std::numeric_limits<int32_t>::min()};
const float kF32[] = {0.f, 0.1f, 0.5f, 0.999f, 1.f, -0.1f, 1e-5f, 2.f,
                      std::numeric_limits<float>::infinity(),
                      std::numeric_limits<float>::quiet_NaN()};

void mutate(bpt_layer_desc& d) {
  switch (next_u64() % 20) {
    case 0: d.abi_version = pick(kI32); break;
    case 1: d.dtype = pick(kI32); break;
    case 2: d.norm = pick(kI32); break;
    case 3: d.ffn = pick(kI32); break;
    case 4: d.causal = pick(kI32); break;
    case 5: d.use_rope = pick(kI32); break;
    case 6: d.batch = pick(kI64); break;
    case 7: d.seq_len = pick(kI64); break;
    case 8: d.hidden = pick(kI64); break;
    case 9: d.n_heads = pick(kI64); break;
    case 10: d.n_kv_heads = pick(kI64); break;
    case 11: d.head_dim = pick(kI64); break;
    case 12: d.ffn_dim = pick(kI64); break;
    case 13: d.q_block = pick(kI64); break;
    case 14: d.kv_block = pick(kI64); break;
    case 15: d.head_chunk = pick(kI64); break;
    case 16: d.norm_eps = pick(kF32); break;
    case 17: d.window = pick(kI32); break;
    case 18: d.dropout_p = pick(kF32); break;
    default: d.rope_base = (double)pick(kF32); break;
  }
}

// Aligned, non-NULL host addresses that no call may dereference: every call
// below must be refused by the checks that precede the first launch.
alignas(256) unsigned char dummy[4096];

void check_layer(const bpt_layer_desc& d, long& valid) {
  const bpt_status v = bpt_layer_validate(&d);
  const size_t saved = bpt_layer_saved_size(&d);
  const size_t wf = bpt_layer_workspace_size(&d, 0), wb = bpt_layer_workspace_size(&d, 1);
  if (v == BPT_OK) {
    ++valid;
    expect(saved > 0 && wf > 0 && wb > 0, "sizes of a valid layer", "zero size");
  } else {
    expect(saved == 0 && wf == 0 && wb == 0, "sizes of an invalid layer", bpt_last_error());
  }
  expect(std::strlen(bpt_status_string(v)) > 0, "status string", "empty");
  // Refused before any launch: NULL weights, then a workspace one byte short.
  bpt_layer_weights w;
  std::memset(&w, 0, sizeof w);
  bpt_status r = bpt_layer_forward(&d, dummy, &w, dummy, dummy, dummy, sizeof dummy, nullptr);
  expect(r != BPT_OK && r != BPT_EHIP, "forward with NULL weights", bpt_status_string(r));
  if (v == BPT_OK) {
    w.w_qkv = w.w_o = w.w_1 = w.w_2 = w.n1_g = w.n2_g = dummy;
    if (d.ffn == BPT_SWIGLU) w.w_3 = dummy;
    if (d.norm == BPT_LAYERNORM) w.n1_b = w.n2_b = dummy;
    r = bpt_layer_forward(&d, dummy, &w, dummy, dummy, dummy, wf - 1, nullptr);
    expect(r == BPT_EWORKSPACE, "forward with a short workspace", bpt_status_string(r));
    r = bpt_layer_forward(&d, dummy + 1, &w, dummy, dummy, dummy, wf, nullptr);
    expect(r == BPT_EINVAL, "forward with a misaligned input", bpt_status_string(r));
    bpt_layer_grads g;
    std::memset(&g, 0, sizeof g);  // NULL entries: those gradients are skipped
    r = bpt_layer_backward(&d, dummy, &w, dummy, dummy, dummy, &g, dummy, wb - 1, nullptr);
    expect(r == BPT_EWORKSPACE, "backward with a short workspace", bpt_status_string(r));
    g.dw_o = (float*)(void*)(dummy + 2);
    r = bpt_layer_backward(&d, dummy, &w, dummy, dummy, dummy, &g, dummy, wb, nullptr);
    expect(r == BPT_EINVAL, "backward with a misaligned gradient", bpt_status_string(r));
  }
}

void check_stack(const bpt_layer_desc& layer, int64_t L, int64_t k, long& valid) {
  bpt_stack_desc s;
  std::memset(&s, 0, sizeof s);
  s.layer = layer;
  s.n_layers = L;
  s.checkpoint_every = k;
  const bpt_status v = bpt_stack_validate(&s);
  const size_t saved = bpt_stack_saved_size(&s);
  const size_t wf = bpt_stack_workspace_size(&s, 0), wb = bpt_stack_workspace_size(&s, 1);
  if (v == BPT_OK) {
    ++valid;
    expect(wf > 0 && wb > 0, "sizes of a valid stack", "zero size");
    (void)saved;
  } else {
    expect(saved == 0 && wf == 0 && wb == 0, "sizes of an invalid stack", bpt_last_error());
  }
  const bpt_status r =
      bpt_stack_forward(&s, dummy, nullptr, dummy, dummy, dummy, sizeof dummy, nullptr);
  expect(r != BPT_OK && r != BPT_EHIP, "stack forward with NULL weights", bpt_status_string(r));
}

void check_lm(int64_t rows, int64_t h, int64_t V, int64_t chunk, int32_t dtype, long& valid) {
  bpt_lm_head_desc d;
  std::memset(&d, 0, sizeof d);
  d.abi_version = BPT_ABI_VERSION;
  d.dtype = dtype;
  d.rows = rows;
  d.hidden = h;
  d.vocab = V;
  d.chunk_rows = chunk;
  const bpt_status v = bpt_lm_head_validate(&d);
  const size_t saved = bpt_lm_head_saved_size(&d);
  const size_t wf = bpt_lm_head_workspace_size(&d, 0), wb = bpt_lm_head_workspace_size(&d, 1);
  const size_t wfb = bpt_lm_head_workspace_size(&d, 2);
  expect(bpt_lm_head_workspace_size(&d, 3) == 0 && bpt_lm_head_workspace_size(&d, -1) == 0,
         "LM head workspace of an unknown mode", "non-zero");
  if (v == BPT_OK) {
    ++valid;
    expect(saved > 0 && wf > 0 && wb > 0 && wfb > wf + wb, "sizes of a valid LM head",
           "zero size");
    bpt_status r = bpt_lm_head_forward(&d, dummy, dummy, nullptr, (float*)(void*)dummy, dummy, dummy, wf,
                                       nullptr);
    expect(r == BPT_EINVAL, "LM head forward with NULL targets", bpt_status_string(r));
    float* fd = (float*)(void*)dummy;
    r = bpt_lm_head_forward_backward(&d, dummy, dummy, (const int32_t*)(void*)dummy, fd, fd,
                                     nullptr, nullptr, nullptr, 0, dummy, wfb, nullptr);
    expect(r == BPT_EINVAL, "fused LM head with neither dz nor dw_head", bpt_status_string(r));
    r = bpt_lm_head_forward_backward(&d, dummy, dummy, (const int32_t*)(void*)dummy, fd, fd,
                                     nullptr, dummy, nullptr, 0, dummy, wfb - 1, nullptr);
    expect(r == BPT_EWORKSPACE, "fused LM head with a short workspace", bpt_status_string(r));
    r = bpt_lm_head_forward_backward(&d, dummy, dummy, (const int32_t*)(void*)dummy, fd, fd,
                                     nullptr, dummy, nullptr, 2, dummy, wfb, nullptr);
    expect(r == BPT_EINVAL, "fused LM head with accumulate = 2", bpt_status_string(r));
  } else {
    expect(saved == 0 && wf == 0 && wb == 0 && wfb == 0, "sizes of an invalid LM head",
           bpt_last_error());
    const bpt_status r = bpt_lm_head_forward_backward(&d, dummy, dummy, nullptr, nullptr, nullptr,
                                                      nullptr, dummy, nullptr, 0, dummy,
                                                      sizeof dummy, nullptr);
    expect(r != BPT_OK && r != BPT_EHIP, "fused LM head with an invalid descriptor",
           bpt_status_string(r));
  }
}

}  // namespace

int main() {
  long n = 0, valid = 0, svalid = 0, lvalid = 0;
  // Single-field and multi-field mutations of a valid descriptor.
  for (int i = 0; i < 20000; ++i) {
    bpt_layer_desc d = base_desc();
    const int muts = 1 + (int)(next_u64() % 3);
    for (int m = 0; m < muts; ++m) mutate(d);
    check_layer(d, valid);
    ++n;
    if (i % 10 == 0) check_stack(d, pick(kI64), pick(kI64), svalid);
  }
  // Valid families: every dtype / norm / FFN / GQA / window / dropout mix.
  for (int dt = 0; dt < 2; ++dt)
    for (int nm = 0; nm < 2; ++nm)
      for (int ff = 0; ff < 3; ++ff)
        for (int kv : {16, 4, 1})
          for (int win : {0, 1, 100, 1 << 20})
            for (float p : {0.f, 0.1f}) {
              bpt_layer_desc d = base_desc();
              d.dtype = dt;
              d.norm = nm;
              d.ffn = ff;
              d.n_kv_heads = kv;
              d.head_chunk = kv == 16 ? 4 : 16;
              d.window = win;
              d.dropout_p = p;
              d.use_rope = kv != 16;
              check_layer(d, valid);
              ++n;
              for (int64_t L : {1, 3, 8})
                for (int64_t k : {0, 1, 2, 3, 8}) check_stack(d, L, k, svalid);
            }
  for (int i = 0; i < 5000; ++i)
    check_lm(pick(kI64), pick(kI64), pick(kI64), pick(kI64), (int32_t)(next_u64() % 3), lvalid);
  check_lm(131072, 2048, 50304, 8192, BPT_BF16, lvalid);
  check_lm(1000, 256, 1024, 256, BPT_F32, lvalid);
  for (int c = -2; c < 12; ++c) expect(bpt_status_string((bpt_status)c) != nullptr, "status", "");
  std::printf("checked %ld layer descriptors (%ld valid), stacks %ld valid, LM heads %ld valid; "
              "%d failures\n",
              n, valid, svalid, lvalid, failures);
  return failures == 0 ? 0 : 1;
}
