// Drives the C ABI of the emulated library inside a process built with
// AddressSanitizer and UndefinedBehaviorSanitizer (TEST INFRASTRUCTURE ONLY;
// built by tests/emu/sanitize.py).  No Python runs in this process, so the
// sanitizers see the engine's host code and the kernels' emulated code
// alone.
//
// Usage: san_driver CASE_FILE
// The case file (little-endian, written by the test) holds: 14 int32/float
// words of gpt2_config in declaration order, then int32 B, T, micro, steps,
// float lr, then steps * micro * 2 arrays of B*T int32 (tokens, targets).
// For every optimizer step the driver prints "step K loss L norm N".  It
// also exercises the host-side checks (bad configs and arguments, call
// order, token range, arena guards, step count, the single-block call) and
// exits non-zero on any unexpected status.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gpt2.h"

#define EXPECT(cond)                                                           \
  do {                                                                         \
    if (!(cond)) {                                                             \
      std::fprintf(stderr, "san_driver: check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(3);                                                            \
    }                                                                          \
  } while (0)

static void* arena(size_t n) { return std::aligned_alloc(256, (n + 255) / 256 * 256); }

static void host_only_checks(const gpt2_config& good) {
  gpt2_config bad = good;
  bad.n_embd = 65;
  EXPECT(gpt2_arena_bytes(&bad) == 0);
  EXPECT(gpt2_arena_bytes(nullptr) == 0);
  bad = good;
  bad.max_seq = bad.block_size + 1;
  EXPECT(gpt2_num_params(&bad) == -1);
  EXPECT(std::isnan(gpt2_lr_at(-1, 6e-4, 6e-5, 132, 3400)));
  EXPECT(gpt2_lr_at(132, 6e-4, 6e-5, 132, 3400) == 6e-4);
  std::vector<float> p((size_t)gpt2_num_params(&good));
  EXPECT(gpt2_init_host(&good, 3, p.data()) == GPT2_OK);
  EXPECT(gpt2_init_host(&good, 3, nullptr) == GPT2_E_ARG);
  gpt2_ctx* c = nullptr;
  EXPECT(gpt2_create(&good, 0, nullptr, 1 << 20, nullptr, &c) == GPT2_E_ARENA);
  EXPECT(gpt2_create(&good, 0, (void*)256, 16, nullptr, &c) == GPT2_E_ARENA);
  EXPECT(gpt2_create(&bad, 0, (void*)256, 1ull << 40, nullptr, &c) == GPT2_E_ARG);
  EXPECT(gpt2_create(&good, 0, nullptr, 0, nullptr, nullptr) == GPT2_E_ARG);
}

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  gpt2_config cfg;
  int32_t hdr[4];
  float lr;
  EXPECT(std::fread(&cfg, sizeof(cfg), 1, f) == 1);
  EXPECT(std::fread(hdr, sizeof(hdr), 1, f) == 1);
  EXPECT(std::fread(&lr, sizeof(lr), 1, f) == 1);
  const int B = hdr[0], T = hdr[1], micro = hdr[2], steps = hdr[3];
  const size_t n = (size_t)B * T;
  std::vector<std::vector<int32_t>> tok, tgt;
  for (int i = 0; i < steps * micro; ++i) {
    tok.emplace_back(n);
    tgt.emplace_back(n);
    EXPECT(std::fread(tok.back().data(), 4, n, f) == n);
    EXPECT(std::fread(tgt.back().data(), 4, n, f) == n);
  }
  std::fclose(f);

  host_only_checks(cfg);

  const size_t nbytes = gpt2_arena_bytes(&cfg);
  EXPECT(nbytes > 0);
  void* a = arena(nbytes);
  gpt2_ctx* c = nullptr;
  EXPECT(gpt2_create(&cfg, 0, a, nbytes, nullptr, &c) == GPT2_OK);
  EXPECT(gpt2_backward(c, 1.f) == GPT2_E_STATE);
  EXPECT(gpt2_step(c, lr, 1.f, nullptr) == GPT2_E_STATE);
  EXPECT(gpt2_forward(c, tok[0].data(), tgt[0].data(), B + 1, T, nullptr) == GPT2_E_SHAPE);
  std::vector<int32_t> badtok = tok[0];
  badtok[n / 2] = cfg.vocab_size;
  float loss = 0.f, norm = 0.f;
  EXPECT(gpt2_forward(c, badtok.data(), tgt[0].data(), B, T, &loss) == GPT2_E_TOKEN);
  EXPECT(gpt2_check_arena(c, nullptr) == GPT2_OK);

  for (int s = 0; s < steps; ++s) {
    double lsum = 0.0;
    for (int k = 0; k < micro; ++k) {
      const int i = s * micro + k;
      EXPECT(gpt2_forward(c, tok[i].data(), tgt[i].data(), B, T, &loss) == GPT2_OK);
      lsum += loss;
      EXPECT(gpt2_backward(c, 1.f / (float)micro) == GPT2_OK);
    }
    EXPECT(gpt2_step(c, lr, 1.f, &norm) == GPT2_OK);
    std::printf("step %d loss %.9g norm %.9g\n", s, lsum / micro, (double)norm);
  }
  int32_t nbad = -1;
  EXPECT(gpt2_check_arena(c, &nbad) == GPT2_OK && nbad == 0);
  int64_t t = -1;
  EXPECT(gpt2_get_step_count(c, &t) == GPT2_OK && t == steps);
  EXPECT(gpt2_set_step_count(c, -1) == GPT2_E_ARG);
  EXPECT(gpt2_set_step_count(c, 5) == GPT2_OK);
  EXPECT(gpt2_get_step_count(c, &t) == GPT2_OK && t == 5);
  EXPECT(gpt2_sync_weight_copies(c) == GPT2_OK);
  EXPECT(gpt2_timing_enable(c, 99) == GPT2_E_ARG);
  EXPECT(gpt2_timing_enable(c, GPT2_T_GEMM) == GPT2_OK);

  // one block in isolation (fp32 host buffers of [B, T, C])
  const size_t nx = n * cfg.n_embd;
  std::vector<float> x(nx), dy(nx), y(nx), dx(nx);
  for (size_t i = 0; i < nx; ++i) {
    x[i] = std::sin(0.37 * (double)i);
    dy[i] = 1e-3f * std::cos(0.11 * (double)i);
  }
  EXPECT(gpt2_block_fwd_bwd(c, 0, x.data(), dy.data(), y.data(), dx.data(), B, T) == GPT2_OK);
  double ms = 0.0;
  int64_t launches = 0;
  EXPECT(gpt2_timing_read(c, &ms, &launches) == GPT2_OK && launches == 12);  // 4 forward + 8 backward GEMMs
  for (size_t i = 0; i < nx; ++i) EXPECT(std::isfinite(y[i]) && std::isfinite(dx[i]));
  EXPECT(gpt2_block_fwd_bwd(c, cfg.n_layer, x.data(), dy.data(), y.data(), dx.data(), B, T) == GPT2_E_ARG);
  EXPECT(gpt2_check_arena(c, &nbad) == GPT2_OK);

  gpt2_tensor_desc d;
  const int32_t nt = gpt2_num_tensors(c);
  EXPECT(nt > 0);
  for (int32_t i = 0; i < nt; ++i) EXPECT(gpt2_tensor_info(c, i, &d) == GPT2_OK && d.offset + d.bytes <= nbytes);
  EXPECT(gpt2_tensor_info(c, nt, &d) == GPT2_E_ARG);
  gpt2_destroy(c);
  std::free(a);
  std::printf("done\n");
  return 0;
}
