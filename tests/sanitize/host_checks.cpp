// Host-side argument checks of the C ABI, for a build of m2_api.cpp under AddressSanitizer:
// every call below is rejected on the host before any HIP call, so the program runs without
// a GPU. Fake device pointers are 16-byte aligned non-null addresses that no check
// dereferences. Prints one line per failed expectation; the exit status is their number.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "m2.h"

namespace {

int g_fail = 0;

void expect(int got, int want, const char *what) {
  if (got != want) {
    std::printf("FAIL %s: got %d, want %d (%s)\n", what, got, want, m2_last_error());
    ++g_fail;
  }
}

void *fake(uintptr_t k = 1) { return reinterpret_cast<void *>(0x10000u * k); }

m2_config good_cfg(int wtype = M2_W_BF16) {
  m2_config c{};
  c.d_model = 256;
  c.n_heads = 8;
  c.head_dim = 32;
  c.d_state = 16;
  c.n_groups = 2;
  c.d_conv = 4;
  c.norm_group = 0;
  c.norm_eps = 1e-5f;
  c.wtype = wtype;
  c.q_group = wtype == M2_W_INT8G ? 64 : 64;
  c.q_gamma_in = 1.0f;
  c.q_gamma_out = 1.0f;
  return c;
}

m2_weights fake_weights(bool scales) {
  m2_weights w{};
  w.w_in = fake(1);
  w.w_out = fake(2);
  w.conv_w = static_cast<const float *>(fake(3));
  w.conv_b = static_cast<const float *>(fake(4));
  w.dt_bias = static_cast<const float *>(fake(5));
  w.A_log = static_cast<const float *>(fake(6));
  w.D = static_cast<const float *>(fake(7));
  w.norm_w = static_cast<const float *>(fake(8));
  if (scales) {
    w.s_in = fake(9);
    w.s_out = fake(10);
  }
  return w;
}

}  // namespace

int main() {
  expect(m2_abi_version(), M2_ABI_VERSION, "abi version");

  // layer creation
  m2_layer lay = nullptr;
  m2_config c = good_cfg();
  m2_weights w = fake_weights(false);
  expect(m2_layer_create(&c, &w, nullptr), M2_ERR_NULL, "create: out NULL");
  expect(m2_layer_create(nullptr, &w, &lay), M2_ERR_NULL, "create: cfg NULL");
  expect(m2_layer_create(&c, nullptr, &lay), M2_ERR_NULL, "create: weights NULL");
  const struct { int field; int value; } bad[] = {{0, 0}, {0, 250}, {1, 0}, {2, 30}, {3, 0}, {4, 3},
                                                 {5, 1}, {5, 9}, {6, 6}, {8, 9}};
  for (const auto &b : bad) {
    m2_config x = good_cfg();
    int32_t *f[] = {&x.d_model, &x.n_heads, &x.head_dim, &x.d_state, &x.n_groups, &x.d_conv, &x.norm_group,
                    nullptr, &x.wtype};
    *f[b.field] = b.value;
    const int rc = m2_layer_create(&x, &w, &lay);
    if (rc >= 0) {
      std::printf("FAIL create accepted field %d = %d\n", b.field, b.value);
      ++g_fail;
      m2_layer_destroy(lay);
    }
  }
  m2_weights wn = fake_weights(false);
  wn.w_out = nullptr;
  expect(m2_layer_create(&c, &wn, &lay), M2_ERR_NULL, "create: w_out NULL");
  m2_weights wa = fake_weights(false);
  wa.w_in = static_cast<const char *>(fake(1)) + 8;
  expect(m2_layer_create(&c, &wa, &lay), M2_ERR_ALIGN, "create: w_in misaligned");
  m2_config ci = good_cfg(M2_W_INT8G);
  expect(m2_layer_create(&ci, &w, &lay), M2_ERR_NULL, "create: int8 without scales");
  m2_config cf = good_cfg(M2_W_F32);
  m2_weights wp = fake_weights(false);
  wp.w_in_panels = fake(11);
  expect(m2_layer_create(&cf, &wp, &lay), M2_ERR_DTYPE, "create: panels with f32 weights");
  wp.w_out_panels = static_cast<const char *>(fake(12)) + 8;
  expect(m2_layer_create(&c, &wp, &lay), M2_ERR_ALIGN, "create: misaligned panels");
  expect(m2_layer_create(&c, &w, &lay), M2_OK, "create: good layer");

  // state and step checks (nothing is launched)
  size_t ssm_b = 0, conv_b = 0;
  expect(m2_state_sizes(&c, 0, &ssm_b, &conv_b), M2_ERR_SHAPE, "state sizes: 0 slots");
  expect(m2_state_sizes(&c, 4, &ssm_b, &conv_b), M2_OK, "state sizes");
  expect(ssm_b == (size_t)4 * 8 * 32 * 16 * 4 ? 0 : 1, 0, "state sizes: ssm bytes");
  m2_state st = nullptr;
  expect(m2_state_create(lay, 4, nullptr, static_cast<float *>(fake(13)), &st), M2_ERR_NULL, "state: ssm NULL");
  expect(m2_state_create(lay, 4, static_cast<float *>(fake(13)), static_cast<float *>(fake(14)), &st), M2_OK,
         "state: good");
  float *x = static_cast<float *>(fake(15)), *y = static_cast<float *>(fake(16));
  void *ws = fake(17);
  const size_t wsb = m2_step_workspace(lay, 3);
  expect(wsb > 0 ? 0 : 1, 0, "step workspace size");
  expect(m2_step(nullptr, st, x, y, 1, nullptr, 0, ws, wsb, nullptr), M2_ERR_NULL, "step: layer NULL");
  expect(m2_step(lay, st, x, y, 0, nullptr, 0, ws, wsb, nullptr), M2_ERR_SHAPE, "step: batch 0");
  expect(m2_step(lay, st, x, y, 5, nullptr, 0, ws, 1u << 30, nullptr), M2_ERR_SLOT, "step: batch > slots");
  expect(m2_step(lay, st, x + 1, y, 1, nullptr, 0, ws, wsb, nullptr), M2_ERR_ALIGN, "step: x misaligned");
  expect(m2_step(lay, st, x, x, 1, nullptr, 0, ws, wsb, nullptr), M2_ERR_SHAPE, "step: y aliases x");
  expect(m2_step(lay, st, x, y, 1, nullptr, 8, ws, wsb, nullptr), M2_ERR_UNSUPPORTED, "step: unknown flag");
  expect(m2_step(lay, st, x, y, 3, nullptr, 0, ws, wsb - 1, nullptr), M2_ERR_WORKSPACE, "step: workspace short");
  expect(m2_step_noalloc(lay, st, x, y, 5, nullptr, 0, nullptr), M2_ERR_SLOT, "noalloc: batch > slots");
  expect(m2_prefill(lay, st, x, y, 1, 16, 15, nullptr, 0, ws, 1u << 30, nullptr) < 0 ? 0 : 1, 0,
         "prefill: chunk not a multiple of 16");
  expect(m2_step_plan(nullptr, 1), -1, "plan: layer NULL");

  // panels
  expect(m2_pack_panels(M2_W_F32, fake(1), 16, 32, fake(2), nullptr), M2_ERR_DTYPE, "panels: f32");
  expect(m2_pack_panels(M2_W_BF16, fake(1), 0, 32, fake(2), nullptr), M2_ERR_SHAPE, "panels: 0 rows");
  expect(m2_pack_panels(M2_W_BF16, nullptr, 16, 32, fake(2), nullptr), M2_ERR_NULL, "panels: w NULL");
  expect(m2_pack_panels(M2_W_BF16, fake(1), 16, 32, static_cast<char *>(fake(2)) + 4, nullptr), M2_ERR_ALIGN,
         "panels: out misaligned");
  expect(m2_panels_bytes(M2_W_BF16, 37, 100) == 3u * 4 * 64 * 16 ? 0 : 1, 0, "panels: size");

  // heads
  m2_head_config hc{4480, 1000, M2_W_BF16, 0, 1.0f};
  expect(m2_head_workspace(&hc, 1) > 0 ? 0 : 1, 0, "head workspace");
  m2_head_config hb = hc;
  hb.d_model = 4484;
  expect(m2_head_workspace(&hb, 1) == 0 ? 0 : 1, 0, "head: d_model not a multiple of 8");
  int32_t *tok = static_cast<int32_t *>(fake(18));
  expect(m2_head_argmax(&hc, nullptr, nullptr, x, 1, tok, nullptr, ws, 1u << 30, nullptr), M2_ERR_NULL,
         "head: w NULL");

  // attention
  m2_attn_config ac{256, 4, 2, 64, 80, M2_W_BF16, 0, 1.0f, 1.0f};
  m2_attn_weights aw{fake(1), nullptr, fake(2), nullptr};
  m2_attn at = nullptr;
  m2_attn_config ab = ac;
  ab.head_dim = 96;
  expect(m2_attn_create(&ab, &aw, &at) < 0 ? 0 : 1, 0, "attn: head_dim 96");
  ab = ac;
  ab.n_q = 3;
  expect(m2_attn_create(&ab, &aw, &at) < 0 ? 0 : 1, 0, "attn: n_q not a multiple of n_kv");
  expect(m2_attn_create(&ac, &aw, &at), M2_OK, "attn: good");

  // stack
  m2_stack sk = nullptr;
  m2_stack_layer tab[2] = {{M2_LAYER_MIXER, lay, st, nullptr, nullptr, nullptr},
                           {M2_LAYER_ATTN, at, nullptr, fake(19), fake(20), static_cast<int32_t *>(fake(21))}};
  expect(m2_stack_create(tab, 2, 8, &sk) < 0 ? 0 : 1, 0, "stack: more slots than the mixer state has");
  m2_stack_layer bad_tab[1] = {{7, lay, st, nullptr, nullptr, nullptr}};
  expect(m2_stack_create(bad_tab, 1, 4, &sk) < 0 ? 0 : 1, 0, "stack: unknown kind");
  tab[1].k_cache = static_cast<char *>(fake(19)) + 4;
  expect(m2_stack_create(tab, 2, 4, &sk), M2_ERR_ALIGN, "stack: misaligned k cache");
  tab[1].k_cache = fake(19);
  expect(m2_stack_create(tab, 2, 4, &sk), M2_OK, "stack: good");
  expect(m2_stack_step(sk, x, y, 0, nullptr, ws, 1u << 30, nullptr) < 0 ? 0 : 1, 0, "stack step: batch 0");
  // the persistent stack step's entry points: workspace, run count and the checks before
  // any launch (no GPU here, so the persistent path never applies)
  const size_t need_p = m2_stack_workspace_flags(sk, 1, M2_PERSISTENT);
  expect(need_p > m2_stack_workspace(sk, 1) ? 0 : 1, 0, "stack: persistent area in the workspace");
  expect(m2_stack_workspace_flags(sk, 1, 8) == 0 ? 0 : 1, 0, "stack workspace: unknown flag");
  expect(m2_stack_persistent_runs(sk, 1, M2_PERSISTENT), 0, "stack: no persistent run without a GPU");
  expect(m2_stack_persistent_runs(nullptr, 1, M2_PERSISTENT), -1, "stack runs: NULL stack");
  expect(m2_stack_step_flags(sk, x, y, 1, nullptr, 8, ws, need_p, nullptr), M2_ERR_UNSUPPORTED,
         "stack step: unknown flag");
  expect(m2_stack_step_flags(sk, x, y, 1, nullptr, M2_PERSISTENT, ws, need_p - 1, nullptr), M2_ERR_WORKSPACE,
         "stack step: persistent workspace one byte short");
  expect(m2_stack_step_flags(sk, x, y, 5, nullptr, M2_PERSISTENT, ws, need_p, nullptr), M2_ERR_SLOT,
         "stack step: more sessions than slots");
  m2_stack_destroy(sk);

  m2_attn_destroy(at);
  m2_state_destroy(st);
  m2_layer_destroy(lay);
  std::printf("%d failed\n", g_fail);
  return g_fail;
}
