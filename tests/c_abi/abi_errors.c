/*
 * A C program built against include/ddtree.h with the C compiler: it checks that the header is
 * plain C, that the library links from C, and that every entry point rejects invalid arguments
 * with the documented DDTREE_ERR_* code before anything is launched.  No call here reaches the
 * GPU: every argument list fails host-side validation, which reads no device memory, so the
 * pointers are fake (distinct, aligned, never dereferenced).  Exit status 0 when every check
 * holds; each failed check prints one line.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ddtree.h"

static int failures = 0;
static int checks = 0;

static void expect(const char* what, long long got, long long want) {
  ++checks;
  if (got != want) {
    ++failures;
    printf("FAIL %s: got %lld, want %lld\n", what, got, want);
  }
}

/* Fake device addresses: far apart, 256-byte aligned, never dereferenced. */
static void* fake(int i) { return (void*)(uintptr_t)(0x100000000ull + (uint64_t)i * 0x40000000ull); }
static void* misaligned(int i) { return (void*)((char*)fake(i) + 2); }

int main(void) {
  void *q_lat = fake(1), *q_pe = fake(2), *ckv = fake(3), *kpe = fake(4);
  int32_t* parents = (int32_t*)fake(5);
  float *out = (float*)fake(6), *lse = (float*)fake(7);
  void* ws = fake(8);
  int32_t* status = (int32_t*)fake(9);
  int32_t *keep = (int32_t*)fake(10), *n_keep = (int32_t*)fake(11), *next_tok = (int32_t*)fake(12);
  int32_t *draft = (int32_t*)fake(13), *target = (int32_t*)fake(14), *plens = (int32_t*)fake(15);
  hipStream_t stream = NULL;

  /* version and status strings */
  expect("version", ddtree_version(), DDTREE_VERSION);
  {
    const int codes[] = {DDTREE_OK, DDTREE_ERR_NULL, DDTREE_ERR_SHAPE, DDTREE_ERR_ALIGN, DDTREE_ERR_ALIAS,
                         DDTREE_ERR_WORKSPACE, DDTREE_ERR_HIP};
    for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
      const char* s = ddtree_status_string(codes[i]);
      expect("status string present", s != NULL && strlen(s) > 0, 1);
    }
    expect("unknown status string", strcmp(ddtree_status_string(-99), "unknown status") == 0, 1);
  }

  /* ddtree_verify_attn */
  expect("verify NULL q_lat", ddtree_verify_attn(NULL, q_pe, ckv, kpe, 16, parents, 9, 1, out, lse, stream),
         DDTREE_ERR_NULL);
  expect("verify NULL lse", ddtree_verify_attn(q_lat, q_pe, ckv, kpe, 16, parents, 9, 1, out, NULL, stream),
         DDTREE_ERR_NULL);
  expect("verify q_len 0", ddtree_verify_attn(q_lat, q_pe, ckv, kpe, 16, parents, 0, 1, out, lse, stream),
         DDTREE_ERR_SHAPE);
  expect("verify q_len 65", ddtree_verify_attn(q_lat, q_pe, ckv, kpe, 16, parents, 65, 1, out, lse, stream),
         DDTREE_ERR_SHAPE);
  expect("verify 0 streams", ddtree_verify_attn(q_lat, q_pe, ckv, kpe, 16, parents, 9, 0, out, lse, stream),
         DDTREE_ERR_SHAPE);
  expect("verify negative prefix", ddtree_verify_attn(q_lat, q_pe, ckv, kpe, -1, parents, 9, 1, out, lse, stream),
         DDTREE_ERR_SHAPE);
  expect("verify misaligned ckv",
         ddtree_verify_attn(q_lat, q_pe, misaligned(3), kpe, 16, parents, 9, 1, out, lse, stream), DDTREE_ERR_ALIGN);
  expect("verify out aliases q_lat",
         ddtree_verify_attn(q_lat, q_pe, ckv, kpe, 16, parents, 9, 1, (float*)q_lat, lse, stream), DDTREE_ERR_ALIAS);

  /* ddtree_verify_attn_ex and the size queries */
  expect("ex kv_rows too small",
         ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, 16, parents, 9, 1, out, lse, 24, 0.f, 0, ws, 1 << 20, status,
                               stream),
         DDTREE_ERR_SHAPE);
  expect("ex negative splits",
         ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, 16, parents, 9, 1, out, lse, 25, 0.f, -1, ws, 1 << 20, status,
                               stream),
         DDTREE_ERR_SHAPE);
  expect("ex misaligned status",
         ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, 16, parents, 9, 1, out, lse, 25, 0.f, 0, ws, 1 << 20,
                               (int32_t*)((char*)status + 1), stream),
         DDTREE_ERR_ALIGN);
  {
    const size_t need = ddtree_verify_attn_workspace_size(4096, 33, 1, 8);
    expect("workspace size for 8 splits > 0", need > 0, 1);
    expect("ex workspace missing",
           ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, 4096, parents, 33, 1, out, lse, 4129, 0.f, 8, NULL, 0,
                                 status, stream),
           DDTREE_ERR_WORKSPACE);
    expect("ex workspace too small",
           ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, 4096, parents, 33, 1, out, lse, 4129, 0.f, 8, ws, need - 1,
                                 status, stream),
           DDTREE_ERR_WORKSPACE);
    expect("ex workspace aliases out",
           ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, 4096, parents, 33, 1, out, lse, 4129, 0.f, 8, out, need,
                                 status, stream),
           DDTREE_ERR_ALIAS);
  }
  expect("workspace size, one split", (long long)ddtree_verify_attn_workspace_size(4096, 33, 1, 1), 0);
  expect("workspace size, bad shape", (long long)ddtree_verify_attn_workspace_size(16, 0, 1, 0), 0);
  expect("num splits, forced 1", ddtree_verify_attn_num_splits(4096, 33, 64, 1), 1);
  expect("num splits, forced 8", ddtree_verify_attn_num_splits(4096, 33, 1, 8), 8);
  expect("num splits, bad shape", ddtree_verify_attn_num_splits(16, 65, 1, 0), DDTREE_ERR_SHAPE);

  /* ddtree_verify_attn_noalloc: validated like the _ex call; a forced plan whose partials do not
     fit the library's scratch array is refused before anything is launched */
  expect("noalloc NULL parents",
         ddtree_verify_attn_noalloc(q_lat, q_pe, ckv, kpe, 16, NULL, 9, 1, out, lse, 25, 0.f, 0, status, stream),
         DDTREE_ERR_NULL);
  expect("noalloc forced plan beyond the scratch",
         ddtree_verify_attn_workspace_size(4096, 33, 64, 64) > DDTREE_NOALLOC_SCRATCH_BYTES, 1);
  expect("noalloc refuses it",
         ddtree_verify_attn_noalloc(q_lat, q_pe, ckv, kpe, 4096, parents, 33, 64, out, lse, 4129, 0.f, 64, status,
                                    stream),
         DDTREE_ERR_WORKSPACE);

  /* ddtree_verify_attn_ragged */
  expect("ragged NULL prefix_lens",
         ddtree_verify_attn_ragged(q_lat, q_pe, ckv, kpe, NULL, 16, parents, 9, 1, out, lse, 25, 0.f, 1, NULL, 0,
                                   status, stream),
         DDTREE_ERR_NULL);
  expect("ragged prefix_lens aliases out",
         ddtree_verify_attn_ragged(q_lat, q_pe, ckv, kpe, (const int32_t*)out, 16, parents, 9, 1, out, lse, 25, 0.f,
                                   1, NULL, 0, status, stream),
         DDTREE_ERR_ALIAS);

  /* compaction */
  {
    ddtree_kv_cache cache = {ckv, kpe, 25, 1};
    ddtree_kv_cache bad_rows = {ckv, kpe, 0, 1};
    ddtree_kv_cache null_ckv = {NULL, kpe, 25, 1};
    ddtree_kv_cache overlap = {ckv, (char*)ckv + 64, 25, 1};
    expect("compact NULL cache", ddtree_compact_kv(NULL, 16, keep, n_keep, 9, status, stream), DDTREE_ERR_NULL);
    expect("compact NULL ckv", ddtree_compact_kv(&null_ckv, 16, keep, n_keep, 9, status, stream), DDTREE_ERR_NULL);
    expect("compact NULL keep", ddtree_compact_kv(&cache, 16, NULL, n_keep, 9, status, stream), DDTREE_ERR_NULL);
    expect("compact kv_rows 0", ddtree_compact_kv(&bad_rows, 0, keep, n_keep, 9, status, stream), DDTREE_ERR_SHAPE);
    expect("compact prefix past rows", ddtree_compact_kv(&cache, 26, keep, n_keep, 9, status, stream),
           DDTREE_ERR_SHAPE);
    expect("compact keep_stride 0", ddtree_compact_kv(&cache, 16, keep, n_keep, 0, status, stream),
           DDTREE_ERR_SHAPE);
    expect("compact misaligned keep",
           ddtree_compact_kv(&cache, 16, (const int32_t*)((char*)keep + 2), n_keep, 9, status, stream),
           DDTREE_ERR_ALIGN);
    expect("compact ckv overlaps kpe", ddtree_compact_kv(&overlap, 16, keep, n_keep, 9, status, stream),
           DDTREE_ERR_ALIAS);
    expect("compact keep inside the cache",
           ddtree_compact_kv(&cache, 16, (const int32_t*)ckv, n_keep, 9, status, stream), DDTREE_ERR_ALIAS);
    expect("compact_ragged NULL prefix_lens", ddtree_compact_kv_ragged(&cache, NULL, keep, n_keep, 9, status, stream),
           DDTREE_ERR_NULL);

    /* acceptance, alone and fused */
    expect("accept NULL parents",
           ddtree_tree_accept(NULL, draft, target, 9, 1, keep, 9, n_keep, next_tok, status, stream), DDTREE_ERR_NULL);
    expect("accept keep_stride < q_len",
           ddtree_tree_accept(parents, draft, target, 9, 1, keep, 8, n_keep, next_tok, status, stream),
           DDTREE_ERR_SHAPE);
    expect("accept q_len 65",
           ddtree_tree_accept(parents, draft, target, 65, 1, keep, 65, n_keep, next_tok, status, stream),
           DDTREE_ERR_SHAPE);
    expect("accept keep aliases parents",
           ddtree_tree_accept(parents, draft, target, 9, 1, (int32_t*)parents, 9, n_keep, next_tok, status, stream),
           DDTREE_ERR_ALIAS);
    expect("accept misaligned n_keep",
           ddtree_tree_accept(parents, draft, target, 9, 1, keep, 9, (int32_t*)((char*)n_keep + 1), next_tok, status,
                              stream),
           DDTREE_ERR_ALIGN);
    expect("accept_compact NULL cache",
           ddtree_accept_compact(NULL, 16, parents, draft, target, 9, keep, 9, n_keep, next_tok, status, stream),
           DDTREE_ERR_NULL);
    expect("accept_compact tree past the cache",
           ddtree_accept_compact(&cache, 17, parents, draft, target, 9, keep, 9, n_keep, next_tok, status, stream),
           DDTREE_ERR_SHAPE);
    expect("accept_compact_ragged NULL prefix_lens",
           ddtree_accept_compact_ragged(&cache, NULL, parents, draft, target, 9, keep, 9, n_keep, next_tok, status,
                                        stream),
           DDTREE_ERR_NULL);
    expect("accept_compact_ragged prefix_lens inside the cache",
           ddtree_accept_compact_ragged(&cache, (int32_t*)kpe, parents, draft, target, 9, keep, 9, n_keep, next_tok,
                                        status, stream),
           DDTREE_ERR_ALIAS);

    /* every layer's cache */
    ddtree_kv_cache layers[2] = {{ckv, kpe, 25, 1}, {fake(20), fake(21), 25, 1}};
    ddtree_kv_cache same_twice[2] = {{ckv, kpe, 25, 1}, {ckv, kpe, 25, 1}};
    ddtree_kv_cache mixed_rows[2] = {{ckv, kpe, 25, 1}, {fake(20), fake(21), 26, 1}};
    expect("layers NULL table", ddtree_compact_kv_layers(NULL, 2, 16, NULL, keep, n_keep, 9, status, stream),
           DDTREE_ERR_NULL);
    expect("layers 0 layers", ddtree_compact_kv_layers(layers, 0, 16, NULL, keep, n_keep, 9, status, stream),
           DDTREE_ERR_SHAPE);
    expect("layers too many", ddtree_compact_kv_layers(layers, DDTREE_MAX_LAYERS + 1, 16, NULL, keep, n_keep, 9,
                                                       status, stream),
           DDTREE_ERR_SHAPE);
    expect("layers overlapping caches",
           ddtree_compact_kv_layers(same_twice, 2, 16, NULL, keep, n_keep, 9, status, stream), DDTREE_ERR_ALIAS);
    expect("layers misaligned prefix_lens",
           ddtree_compact_kv_layers(layers, 2, 0, (const int32_t*)((char*)plens + 2), keep, n_keep, 9, status, stream),
           DDTREE_ERR_ALIGN);
    expect("layers mixed geometry",
           ddtree_compact_kv_layers(mixed_rows, 2, 16, NULL, keep, n_keep, 9, status, stream), DDTREE_ERR_SHAPE);
    expect("accept_compact_layers NULL draft",
           ddtree_accept_compact_layers(layers, 2, 16, NULL, parents, NULL, target, 9, keep, 9, n_keep, next_tok,
                                        status, stream),
           DDTREE_ERR_NULL);
    expect("accept_compact_layers tree past the cache",
           ddtree_accept_compact_layers(layers, 2, 17, NULL, parents, draft, target, 9, keep, 9, n_keep, next_tok,
                                        status, stream),
           DDTREE_ERR_SHAPE);

    /* tree rows into the cache */
    const float *kv = (const float*)fake(22), *w = (const float*)fake(23);
    const float *cosv = (const float*)fake(24), *sinv = (const float*)fake(25);
    expect("append NULL kv",
           ddtree_append_tree_kv(&cache, 16, NULL, parents, 9, NULL, w, 1e-6f, cosv, sinv, 64, status, stream),
           DDTREE_ERR_NULL);
    expect("append negative eps",
           ddtree_append_tree_kv(&cache, 16, NULL, parents, 9, kv, w, -1.f, cosv, sinv, 64, status, stream),
           DDTREE_ERR_SHAPE);
    expect("append block past the cache",
           ddtree_append_tree_kv(&cache, 17, NULL, parents, 9, kv, w, 1e-6f, cosv, sinv, 64, status, stream),
           DDTREE_ERR_SHAPE);
    expect("append misaligned kv",
           ddtree_append_tree_kv(&cache, 16, NULL, parents, 9, (const float*)misaligned(22), w, 1e-6f, cosv, sinv, 64,
                                 status, stream),
           DDTREE_ERR_ALIGN);
    expect("append kv inside the cache",
           ddtree_append_tree_kv(&cache, 16, NULL, parents, 9, (const float*)ckv, w, 1e-6f, cosv, sinv, 64, status,
                                 stream),
           DDTREE_ERR_ALIAS);
  }

  /* tree build */
  {
    const float* lp = (const float*)fake(30);
    const int32_t* tk = (const int32_t*)fake(31);
    int32_t *bp = (int32_t*)fake(32), *bt = (int32_t*)fake(33), *bn = (int32_t*)fake(34);
    expect("build NULL logprobs",
           ddtree_tree_build(NULL, tk, NULL, 15, 8, 32, 1, bp, bt, bn, NULL, NULL, NULL, NULL, NULL, stream),
           DDTREE_ERR_NULL);
    expect("build budget 64",
           ddtree_tree_build(lp, tk, NULL, 15, 8, 64, 1, bp, bt, bn, NULL, NULL, NULL, NULL, NULL, stream),
           DDTREE_ERR_SHAPE);
    expect("build depth 65",
           ddtree_tree_build(lp, tk, NULL, 65, 8, 32, 1, bp, bt, bn, NULL, NULL, NULL, NULL, NULL, stream),
           DDTREE_ERR_SHAPE);
    expect("build misaligned anc",
           ddtree_tree_build(lp, tk, NULL, 15, 8, 32, 1, bp, bt, bn, NULL, NULL, NULL, NULL,
                             (uint64_t*)((char*)fake(35) + 4), stream),
           DDTREE_ERR_ALIGN);
    expect("build parents alias node_tokens",
           ddtree_tree_build(lp, tk, NULL, 15, 8, 32, 1, bp, bp, bn, NULL, NULL, NULL, NULL, NULL, stream),
           DDTREE_ERR_ALIAS);
  }

  printf("%d checks, %d failed\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
