/*
 * A plain C99 caller of libh2o.so: one layer's cache driven through the C ABI alone.
 * Used by tests/test_gpu_c_driver.py, which compares every result with the same calls made
 * through the Python binding.
 *
 * usage: c_driver DIR B H D KH KL DTYPE T STEPS
 *   DIR holds q_prompt.bin, k_prompt.bin, v_prompt.bin ([B][H][T][D] in DTYPE) and
 *   q_dec.bin, k_dec.bin, v_dec.bin ([STEPS][B][H][D]); the program writes into DIR
 *   prefill_out.bin, colsum.bin, dec_out.bin, victims.bin, ev_pos.bin, ev_acc.bin,
 *   slot_pos.bin, acc.bin, k_slots.bin, v_slots.bin.
 * Exit status: 0, or 1 with a message on stderr.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "h2o.h"

static char dir[4096];

static int fail(const char* what) {
  fprintf(stderr, "c_driver: %s\n", what);
  return 1;
}

static void* read_file(const char* name, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes);
  if (buf && fread(buf, 1, bytes, f) != bytes) {
    free(buf);
    buf = NULL;
  }
  fclose(f);
  return buf;
}

static int write_file(const char* name, const void* dev, size_t bytes) {
  char path[4200];
  void* host = malloc(bytes ? bytes : 1);
  if (!host) return 0;
  if (hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    free(host);
    return 0;
  }
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  int ok = f && fwrite(host, 1, bytes, f) == bytes;
  if (f) fclose(f);
  free(host);
  return ok;
}

/* A device copy of a host file, or NULL. */
static void* upload(const char* name, size_t bytes) {
  void* host = read_file(name, bytes);
  void* dev = NULL;
  if (!host) return NULL;
  if (hipMalloc(&dev, bytes) != hipSuccess ||
      hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess)
    dev = NULL;
  free(host);
  return dev;
}

static void* dalloc(size_t bytes) {
  void* p = NULL;
  return hipMalloc(&p, bytes ? bytes : 16) == hipSuccess ? p : NULL;
}

int main(int argc, char** argv) {
  if (argc != 10) return fail("usage: c_driver DIR B H D KH KL DTYPE T STEPS");
  snprintf(dir, sizeof dir, "%s", argv[1]);
  const int B = atoi(argv[2]), H = atoi(argv[3]), D = atoi(argv[4]);
  const int KH = atoi(argv[5]), KL = atoi(argv[6]), dtype = atoi(argv[7]);
  const int T = atoi(argv[8]), steps = atoi(argv[9]);
  const size_t es = dtype == H2O_F32 ? 4 : 2, units = (size_t)B * H, k = (size_t)(KH + KL);

  h2o_cache_desc c;
  memset(&c, 0, sizeof c);
  c.batch = B;
  c.heads = H;
  c.head_dim = D;
  c.k_heavy = KH;
  c.k_local = KL;
  c.dtype = dtype;
  c.k_slots = dalloc(units * k * D * es);
  c.v_slots = dalloc(units * k * D * es);
  c.slot_pos = (int32_t*)dalloc(units * k * 4);
  c.acc_score = (float*)dalloc(units * k * 4);
  void* q = upload("q_prompt.bin", units * T * D * es);
  void* kp = upload("k_prompt.bin", units * T * D * es);
  void* vp = upload("v_prompt.bin", units * T * D * es);
  void* qd = upload("q_dec.bin", (size_t)steps * units * D * es);
  void* kd = upload("k_dec.bin", (size_t)steps * units * D * es);
  void* vd = upload("v_dec.bin", (size_t)steps * units * D * es);
  float* out_p = (float*)dalloc(units * T * D * 4);
  float* colsum = (float*)dalloc(units * T * 4);
  float* out_d = (float*)dalloc((size_t)steps * units * D * 4);
  int32_t* victims = (int32_t*)dalloc((size_t)steps * units * 4);
  int32_t* ev_pos = (int32_t*)dalloc((size_t)steps * units * 4);
  float* ev_acc = (float*)dalloc((size_t)steps * units * 4);
  if (!c.k_slots || !c.v_slots || !c.slot_pos || !c.acc_score || !q || !kp || !vp || !qd ||
      !kd || !vd || !out_p || !colsum || !out_d || !victims || !ev_pos || !ev_acc)
    return fail("allocation or input file");
  const size_t ws_bytes = h2o_workspace_bytes(&c, T);
  void* ws = ws_bytes ? dalloc(ws_bytes) : NULL;
  if (ws_bytes && !ws) return fail("workspace allocation");

  hipStream_t s;
  if (hipStreamCreate(&s) != hipSuccess) return fail("stream");
  if (h2o_reset(&c, s) != H2O_OK) return fail(h2o_last_error());
  if (h2o_prefill(&c, q, kp, vp, T, out_p, colsum, ws, ws_bytes, s) != H2O_OK)
    return fail(h2o_last_error());
  for (int i = 0; i < steps; ++i) {
    const size_t o = (size_t)i * units;
    h2o_decode_aux aux;
    aux.victim_slot = victims + o;
    aux.evicted_pos = ev_pos + o;
    aux.evicted_acc = ev_acc + o;
    if (h2o_decode_step(&c, (int64_t)T + i, (const char*)qd + o * D * es,
                        (const char*)kd + o * D * es, (const char*)vd + o * D * es,
                        out_d + o * D, &aux, ws, ws_bytes, s) != H2O_OK)
      return fail(h2o_last_error());
  }
  if (hipStreamSynchronize(s) != hipSuccess) return fail("stream synchronize");
  if (!write_file("prefill_out.bin", out_p, units * T * D * 4) ||
      !write_file("colsum.bin", colsum, units * T * 4) ||
      !write_file("dec_out.bin", out_d, (size_t)steps * units * D * 4) ||
      !write_file("victims.bin", victims, (size_t)steps * units * 4) ||
      !write_file("ev_pos.bin", ev_pos, (size_t)steps * units * 4) ||
      !write_file("ev_acc.bin", ev_acc, (size_t)steps * units * 4) ||
      !write_file("slot_pos.bin", c.slot_pos, units * k * 4) ||
      !write_file("acc.bin", c.acc_score, units * k * 4) ||
      !write_file("k_slots.bin", c.k_slots, units * k * D * es) ||
      !write_file("v_slots.bin", c.v_slots, units * k * D * es))
    return fail("output file");
  hipStreamDestroy(s);
  return 0;
}
