// Host driver for the sanitizer test: builds and walks batch-1 plans of the
// tiny, Llama-1B and Llama-8B shapes through mkcheck_walk (planner + address
// walk, host code only) and prints one line per plan.  Built by
// tests/test_host_sanitizers.py with AddressSanitizer and UBSan.
#include <cstdio>
#include <cstring>

#include "../persistent_megakernel_cu_amd/csrc/mk_check.h"

static mk_config shape(int L, int H, int NQ, int NKV, int D, int F, int V, int S, int tied) {
  mk_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = L; c.hidden = H; c.n_heads = NQ; c.n_kv_heads = NKV; c.head_dim = D; c.ffn = F; c.vocab = V;
  c.max_seq = S; c.batch = 1; c.rms_eps = 1e-5f; c.rope_theta = 5e5; c.tie_embeddings = tied;
  return c;
}

int main() {
  struct Case { const char* name; mk_config cfg; int pos; } cases[] = {
      {"tiny", shape(2, 256, 4, 2, 64, 1024, 4096, 48, 1), 47},
      {"llama1b", shape(16, 2048, 32, 8, 64, 8192, 128256, 256, 1), 255},
      {"llama1b-long", shape(16, 2048, 32, 8, 64, 8192, 128256, 8192, 1), 8191},
      {"llama8b", shape(32, 4096, 32, 8, 128, 14336, 128256, 2112, 0), 2049},
  };
  int bad = 0;
  for (const Case& k : cases) {
    mkcheck_report r;
    const int rc = mkcheck_walk(&k.cfg, 256, k.pos, 0, &r);
    std::printf("%s rc=%d checks=%lld violations=%lld %s\n", k.name, rc, r.checks, r.violations, r.first);
    bad += rc != 0 || r.violations != 0;
  }
  return bad;
}
