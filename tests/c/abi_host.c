/* The C ABI used from plain C99: the header compiles as C, and the host-only
 * entry points (version, LPT partition, workspace size, validation with its
 * error message, the per-phase test hook) answer as documented.  Device
 * addresses are plausible values that are never dereferenced; no HIP call is
 * made.  Prints "ok" and exits 0 on success. */
#include <stdio.h>
#include <string.h>

#include "dmuon_ns.h"

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__);       \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static dmuon_tensor fake(int32_t ndim, int64_t b, int64_t r, int64_t c, uintptr_t base) {
  dmuon_tensor t;
  memset(&t, 0, sizeof t);
  t.ndim = ndim;
  if (ndim == 3) {
    t.shape[0] = b; t.shape[1] = r; t.shape[2] = c;
  } else {
    t.shape[0] = r; t.shape[1] = c;
  }
  t.grad_dtype = DMUON_BF16;
  t.grad = (const void*)base;
  t.momentum = (float*)(base + ((uintptr_t)1 << 28));
  t.master = (float*)(base + ((uintptr_t)2 << 28));
  return t;
}

int main(void) {
  CHECK(dmuon_abi_version() == 5);

  /* LPT: 6 matrices over 2 slots, 3 layers (two per layer) */
  {
    const int64_t rows[6] = {64, 64, 32, 32, 16, 16}, cols[6] = {64, 64, 32, 32, 16, 16};
    const int64_t batch[6] = {1, 1, 1, 1, 1, 1};
    const int32_t layer[6] = {0, 0, 1, 1, 2, 2};
    int32_t slot_of[6];
    int64_t load[2], order[6], n_owned = 0, offsets[7];
    int32_t n_groups = 0;
    CHECK(dmuon_lpt_assign(6, rows, cols, batch, layer, 2, 0, 0, slot_of, load, 0, order, &n_owned, offsets,
                           &n_groups) == DMUON_OK);
    CHECK(load[0] + load[1] == 2 * (64 * 64 + 32 * 32 + 16 * 16));
    CHECK(load[0] == load[1]);                     /* one of each layer per slot */
    CHECK(slot_of[0] != slot_of[1] && slot_of[2] != slot_of[3] && slot_of[4] != slot_of[5]);
    CHECK(n_owned == 3 && n_groups == 3);
  }

  /* workspace size, validation and the per-phase hook on plausible addresses */
  {
    const uintptr_t base = (uintptr_t)0x7f0000000000ull;
    dmuon_tensor t[2];
    dmuon_step_cfg cfg;
    size_t bytes = 0;
    dmuon_debug_slice d;
    t[0] = fake(2, 1, 300, 700, base);
    t[1] = fake(3, 2, 600, 280, base + ((uintptr_t)1 << 32));
    memset(&cfg, 0, sizeof cfg);
    cfg.lr = 0.02f; cfg.momentum = 0.95f; cfg.weight_decay = 0.01f; cfg.eps = 1e-7f;
    cfg.a = 3.4445f; cfg.b = -4.775f; cfg.c = 2.0315f; cfg.ns_steps = 5;
    cfg.prec = DMUON_PREC_BF16_MFMA; cfg.grad_scale = 1.0f; cfg.stream_groups = 1;
    CHECK(dmuon_muon_step_workspace_size(t, 2, &cfg, &bytes) == DMUON_OK && bytes > 0);
    {
      const uintptr_t ws = base + ((uintptr_t)1 << 40);
      CHECK(dmuon_debug_slice_buffers(t, 2, &cfg, (void*)ws, bytes, 1, 1, &d) == DMUON_OK);
      CHECK(d.m == 280 && d.n == 600 && d.wide == 0 && d.elem_bytes == 2 && d.ld_m == 320);
      CHECK((uintptr_t)d.a_prime >= ws && (uintptr_t)d.a_prime + (size_t)(d.m * d.ld_m * 2) <= ws + bytes);
      CHECK(dmuon_debug_slice_buffers(t, 2, &cfg, (void*)ws, bytes, 1, 2, &d) == DMUON_E_SHAPE);
      CHECK(strlen(dmuon_last_error()) > 0);
    }
    t[0].ndim = 1;
    CHECK(dmuon_muon_step(t, 2, &cfg, NULL, 0, NULL, NULL, 0) == DMUON_E_NDIM);
    CHECK(strstr(dmuon_last_error(), "2 dims") != NULL);
  }
  printf("ok\n");
  return 0;
}
