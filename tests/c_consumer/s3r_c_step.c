/*
 * A plain C caller of libs3r.so: one decode step's dense verify (with page
 * scores), budget selection, one sparse draft step and the exact accept with its
 * commit, on device buffers this program allocates itself through the HIP
 * runtime. No Python and no torch: it shows the C ABI of include/s3r.h is all a
 * caller needs.
 *
 * Usage: s3r_c_step <dir>
 *   <dir>/meta.txt holds "key value" lines: B Hq Hkv D NB maxp G1 gamma V kv_dtype
 *   logits_dtype max_sel draft_step budget scale temperature (dtypes: 0 fp32,
 *   1 bf16 bit patterns).
 *   Inputs (raw little-endian, row-major, shapes as in include/s3r.h):
 *   k_cache v_cache page_table ctx_lens q_verify q_draft target_logits
 *   draft_logits draft_tokens u_accept u_sample (each "<name>.bin").
 *   Outputs written beside them: verify_out page_scores sel nsel draft_out
 *   num_accepted out_tokens ctx_after (each "<name>.bin").
 * Exit status 0 on success; 1 with a message on stderr otherwise.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "s3r.h"

typedef struct {
  long B, Hq, Hkv, D, NB, maxp, G1, gamma, V, kv_dtype, logits_dtype, max_sel, draft_step;
  double budget, scale, temperature;
} meta_t;

static const char* g_dir;

static int die(const char* what, const char* detail) {
  fprintf(stderr, "s3r_c_step: %s: %s\n", what, detail);
  exit(1);
  return 1;
}

#define HIP_OK(call)                                        \
  do {                                                      \
    hipError_t e_ = (call);                                 \
    if (e_ != hipSuccess) die(#call, hipGetErrorString(e_)); \
  } while (0)

#define S3R_OK(call)                                        \
  do {                                                      \
    s3r_status s_ = (call);                                 \
    if (s_ != S3R_SUCCESS) die(#call, s3r_status_string(s_)); \
  } while (0)

static void path_of(char* out, size_t n, const char* name) { snprintf(out, n, "%s/%s.bin", g_dir, name); }

/* Reads <dir>/<name>.bin, which must hold exactly `bytes` bytes. */
static void* read_input(const char* name, size_t bytes) {
  char path[4096];
  FILE* f;
  void* buf;
  long size;
  path_of(path, sizeof path, name);
  f = fopen(path, "rb");
  if (f == NULL) die("cannot open", path);
  if (fseek(f, 0, SEEK_END) != 0 || (size = ftell(f)) < 0 || fseek(f, 0, SEEK_SET) != 0) die("cannot size", path);
  if ((size_t)size != bytes) die("unexpected size", path);
  buf = malloc(bytes > 0 ? bytes : 1);
  if (buf == NULL) die("out of host memory", path);
  if (bytes > 0 && fread(buf, 1, bytes, f) != bytes) die("short read", path);
  fclose(f);
  return buf;
}

static void write_output(const char* name, const void* p, size_t bytes) {
  char path[4096];
  FILE* f;
  path_of(path, sizeof path, name);
  f = fopen(path, "wb");
  if (f == NULL) die("cannot create", path);
  if (bytes > 0 && fwrite(p, 1, bytes, f) != bytes) die("short write", path);
  if (fclose(f) != 0) die("cannot close", path);
}

/* A device copy of input <name> (bytes long). */
static void* upload(const char* name, size_t bytes) {
  void* h = read_input(name, bytes);
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes > 0 ? bytes : 1));
  HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  free(h);
  return d;
}

static void* device_buffer(size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes > 0 ? bytes : 1));
  return d;
}

static void download(const char* name, const void* d, size_t bytes) {
  void* h = malloc(bytes > 0 ? bytes : 1);
  if (h == NULL) die("out of host memory", name);
  HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  write_output(name, h, bytes);
  free(h);
}

static void read_meta(meta_t* m) {
  char path[4096], key[64];
  double val;
  int seen = 0;
  FILE* f;
  snprintf(path, sizeof path, "%s/meta.txt", g_dir);
  f = fopen(path, "r");
  if (f == NULL) die("cannot open", path);
  memset(m, 0, sizeof *m);
  while (fscanf(f, "%63s %lf", key, &val) == 2) {
    ++seen;
    if (!strcmp(key, "B")) m->B = (long)val;
    else if (!strcmp(key, "Hq")) m->Hq = (long)val;
    else if (!strcmp(key, "Hkv")) m->Hkv = (long)val;
    else if (!strcmp(key, "D")) m->D = (long)val;
    else if (!strcmp(key, "NB")) m->NB = (long)val;
    else if (!strcmp(key, "maxp")) m->maxp = (long)val;
    else if (!strcmp(key, "G1")) m->G1 = (long)val;
    else if (!strcmp(key, "gamma")) m->gamma = (long)val;
    else if (!strcmp(key, "V")) m->V = (long)val;
    else if (!strcmp(key, "kv_dtype")) m->kv_dtype = (long)val;
    else if (!strcmp(key, "logits_dtype")) m->logits_dtype = (long)val;
    else if (!strcmp(key, "max_sel")) m->max_sel = (long)val;
    else if (!strcmp(key, "draft_step")) m->draft_step = (long)val;
    else if (!strcmp(key, "budget")) m->budget = val;
    else if (!strcmp(key, "scale")) m->scale = val;
    else if (!strcmp(key, "temperature")) m->temperature = val;
    else die("unknown key in meta.txt", key);
  }
  fclose(f);
  if (seen != 16) die("meta.txt", "expected 16 keys");
}

int main(int argc, char** argv) {
  meta_t m;
  s3r_paged_kv kv;
  size_t es, ls, ws_verify, ws_accept;
  void *q_verify, *q_draft, *verify_out, *draft_out, *tl, *dl, *ws_v, *ws_a;
  float *scores, *ua, *us;
  int32_t *sel, *nsel, *dtok, *nacc, *otok, *ctx_after;
  if (argc != 2) return die("usage", "s3r_c_step <dir>");
  g_dir = argv[1];
  read_meta(&m);
  es = m.kv_dtype == 1 ? 2 : 4;
  ls = m.logits_dtype == 1 ? 2 : 4;

  memset(&kv, 0, sizeof kv);
  kv.num_blocks = (int32_t)m.NB;
  kv.num_kv_heads = (int32_t)m.Hkv;
  kv.page_size = 16;
  kv.head_dim = (int32_t)m.D;
  kv.max_pages_per_seq = (int32_t)m.maxp;
  kv.dtype = m.kv_dtype == 1 ? S3R_BF16 : S3R_F32;
  kv.k_cache = upload("k_cache", (size_t)m.NB * m.Hkv * 16 * m.D * es);
  kv.v_cache = upload("v_cache", (size_t)m.NB * m.Hkv * m.D * 16 * es);
  kv.page_table = (const int32_t*)upload("page_table", (size_t)m.B * m.maxp * 4);
  kv.ctx_lens = (const int32_t*)upload("ctx_lens", (size_t)m.B * 4);
  q_verify = upload("q_verify", (size_t)m.B * m.G1 * m.Hq * m.D * es);
  q_draft = upload("q_draft", (size_t)m.B * m.Hq * m.D * es);
  tl = upload("target_logits", (size_t)m.B * m.G1 * m.V * ls);
  dl = upload("draft_logits", (size_t)m.B * m.gamma * m.V * ls);
  dtok = (int32_t*)upload("draft_tokens", (size_t)m.B * m.gamma * 4);
  ua = (float*)upload("u_accept", (size_t)m.B * m.gamma * 4);
  us = (float*)upload("u_sample", (size_t)m.B * 4);

  /* dense verify of the block, with the page scores for the next draft */
  verify_out = device_buffer((size_t)m.B * m.G1 * m.Hq * m.D * es);
  scores = (float*)device_buffer((size_t)m.B * m.maxp * 4);
  ws_verify = s3r_dense_verify_workspace_size(&kv, (int32_t)m.B, (int32_t)m.Hq, (int32_t)m.G1);
  ws_v = device_buffer(ws_verify);
  S3R_OK(s3r_dense_verify_attn(&kv, (int32_t)m.B, (int32_t)m.Hq, (int32_t)m.G1, q_verify, (float)m.scale, verify_out,
                               scores, ws_v, ws_verify, NULL));

  /* the budget's top pages of those scores */
  sel = (int32_t*)device_buffer((size_t)m.B * m.max_sel * 4);
  nsel = (int32_t*)device_buffer((size_t)m.B * 4);
  S3R_OK(s3r_select_budget(scores, kv.ctx_lens, (int32_t)m.B, (int32_t)m.maxp, 16, m.budget, sel, nsel,
                           (int32_t)m.max_sel, NULL, 0, NULL));

  /* one sparse draft step over the selected pages and the tail */
  draft_out = device_buffer((size_t)m.B * m.Hq * m.D * es);
  S3R_OK(s3r_sparse_draft_attn(&kv, (int32_t)m.B, (int32_t)m.Hq, (int32_t)m.draft_step, q_draft, (float)m.scale, sel,
                               nsel, (int32_t)m.max_sel, draft_out, NULL, 0, NULL));

  /* exact accept of the drafted block and the commit of the lengths */
  nacc = (int32_t*)device_buffer((size_t)m.B * 4);
  otok = (int32_t*)device_buffer((size_t)m.B * m.G1 * 4);
  ctx_after = (int32_t*)device_buffer((size_t)m.B * 4);
  HIP_OK(hipMemcpy(ctx_after, kv.ctx_lens, (size_t)m.B * 4, hipMemcpyDeviceToDevice));
  ws_accept = s3r_spec_accept_workspace_size((int32_t)m.B, (int32_t)m.gamma, (int32_t)m.V);
  ws_a = device_buffer(ws_accept);
  S3R_OK(s3r_spec_accept((int32_t)m.B, (int32_t)m.gamma, (int32_t)m.V,
                         m.logits_dtype == 1 ? S3R_BF16 : S3R_F32, tl, dl, dtok, ua, us, (float)m.temperature, nacc,
                         otok, ctx_after, ws_a, ws_accept, NULL));
  HIP_OK(hipDeviceSynchronize());

  download("verify_out", verify_out, (size_t)m.B * m.G1 * m.Hq * m.D * es);
  download("page_scores", scores, (size_t)m.B * m.maxp * 4);
  download("sel", sel, (size_t)m.B * m.max_sel * 4);
  download("nsel", nsel, (size_t)m.B * 4);
  download("draft_out", draft_out, (size_t)m.B * m.Hq * m.D * es);
  download("num_accepted", nacc, (size_t)m.B * 4);
  download("out_tokens", otok, (size_t)m.B * m.G1 * 4);
  download("ctx_after", ctx_after, (size_t)m.B * 4);
  printf("s3r_c_step: verify workspace %zu B, accept workspace %zu B: done\n", ws_verify, ws_accept);
  return 0;
}
