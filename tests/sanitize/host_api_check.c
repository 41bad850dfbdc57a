/* Drives the C-ABI's host logic on dry-run handles (no device memory, no GPU) so that a
 * library built with host-side AddressSanitizer and UndefinedBehaviorSanitizer can check
 * it: configs, sizes, the frame sequence (writes, evictions, reads, steps, the zero-copy
 * slot, the sink schedule), snapshots against the closed-form plan, state export/import,
 * batched reads, and the error paths.  Exits non-zero on the first failed expectation; the
 * sanitizers abort on their own findings. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sf.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      exit(1);                                                              \
    }                                                                       \
  } while (0)

static sf_config make(int hw, int x, int y, int w, int heads, int hd, int blocks, int dtype, int sink_gap,
                      int rope_mode, int bias) {
  sf_config c;
  memset(&c, 0, sizeof c);
  c.hw = hw; c.x = x; c.y = y; c.w = w; c.n_heads = heads; c.head_dim = hd; c.n_blocks = blocks;
  c.dtype = dtype; c.max_frames = 0; c.sink_gap = sink_gap; c.rope_theta = 10000.0f; c.rope_mode = rope_mode;
  c.recency_bias = bias;
  return c;
}

/* Snapshot of buf equals the closed-form plan at its current frame. */
static void check_view(const sf_buffer* buf, const sf_config* c) {
  int64_t raw_q[64], sum_q[256], raw_p[64], sum_p[256];
  sf_view q, p;
  memset(&q, 0, sizeof q);
  memset(&p, 0, sizeof p);
  q.raw_frame = raw_q; q.sum_frame = sum_q;
  p.raw_frame = raw_p; p.sum_frame = sum_p;
  EXPECT(c->y + 1 <= 64 && c->w - c->y <= 256);
  EXPECT(sf_query(buf, &q) == SF_OK);
  if (q.t_cur < 0) return;
  EXPECT(sf_plan(c, q.t_cur, &p) == SF_OK);
  EXPECT(p.n_keys == q.n_keys && p.n_seg == q.n_seg && p.raw_slot == q.raw_slot);
  for (int i = 0; i < q.n_seg; ++i) EXPECT(p.seg_begin[i] == q.seg_begin[i] && p.seg_len[i] == q.seg_len[i]);
  for (int i = 0; i <= c->y; ++i) EXPECT(raw_p[i] == raw_q[i]);
  for (int i = 0; i < c->w - c->y; ++i) EXPECT(sum_p[i] == sum_q[i]);
}

/* A dry session through `frames` frames with every call of the sequence. */
static void run_sequence(const sf_config* c, int frames, int use_step) {
  sf_buffer* b = NULL;
  EXPECT(sf_config_check(c) == SF_OK);
  EXPECT(sf_buffer_bytes(c) > 0 && sf_kv_bytes(c) > 0 && sf_kv_bytes(c) <= sf_buffer_bytes(c));
  EXPECT(sf_kv_offset(c, 0, 0) == 0 && sf_kv_offset(c, c->n_blocks - 1, 1) > 0);
  EXPECT(sf_kv_offset(c, c->n_blocks, 0) == -1 && sf_kv_offset(c, 0, 2) == -1);
  EXPECT(sf_buffer_create(c, NULL, 0, NULL, &b) == SF_OK && b != NULL);
  if (c->recency_bias) EXPECT(sf_set_recency_bias(b, NULL, NULL) == SF_OK);
  check_view(b, c);
  for (int64_t t = 0; t < frames; ++t) {
    for (int blk = 0; blk < c->n_blocks; ++blk) {
      if (use_step) {
        EXPECT(sf_step(b, blk, t, NULL, NULL, NULL, NULL, 0.0f, NULL) == SF_OK);
      } else {
        if (blk == 0 && t > 0) EXPECT(sf_evict(b, t, NULL) == SF_OK);
        if (c->rope_mode == SF_ROPE_CALLER && (t % 3) == 1) {
          void *kr = (void*)1, *vr = (void*)1;
          EXPECT(sf_record_slot(b, blk, t, &kr, &vr) == SF_OK && kr == NULL && vr == NULL);
          EXPECT(sf_commit_record(b, blk, t) == SF_OK);
        } else {
          EXPECT(sf_write_record(b, blk, t, NULL, NULL, NULL) == SF_OK);
        }
        sf_buffer* one[1] = {b};
        const void* q[1] = {NULL};
        void* o[1] = {NULL};
        EXPECT(sf_attend(one, 1, blk, q, o, 0.0f, NULL) == SF_OK);
        EXPECT(sf_attend_static_scratch(one, 1, blk, q, o, 0.0f, NULL) == SF_OK);
      }
    }
    check_view(b, c);
    /* out of order: a frame two ahead, a frame behind, a bad block */
    EXPECT(sf_write_record(b, 0, t + 2, NULL, NULL, NULL) == SF_E_ORDER || t + 2 <= t);
    if (t > 0) EXPECT(sf_write_record(b, 0, t - 1, NULL, NULL, NULL) != SF_OK);
    EXPECT(sf_write_record(b, c->n_blocks, t, NULL, NULL, NULL) == SF_E_ARG);
    EXPECT(sf_last_error(b) != NULL && strlen(sf_last_error(b)) > 0);
    check_view(b, c);
  }
  /* state round trip into a second handle */
  const size_t sb = sf_state_bytes(c);
  EXPECT(sb > 0);
  char* st = (char*)malloc(sb);
  EXPECT(st != NULL);
  EXPECT(sf_state_export(b, st, sb) == SF_OK);
  EXPECT(sf_state_export(b, st, sb - 1) == SF_E_ARG);
  sf_buffer* b2 = NULL;
  EXPECT(sf_buffer_create(c, NULL, 0, NULL, &b2) == SF_OK);
  EXPECT(sf_state_import(b2, st, sb - 1) == SF_E_ARG);
  EXPECT(sf_state_import(b2, st, sb) == SF_OK);
  check_view(b2, c);
  /* a batched read over both handles */
  sf_buffer* two[2] = {b, b2};
  const void* q2[2] = {NULL, NULL};
  void* o2[2] = {NULL, NULL};
  EXPECT(sf_attend(two, 2, 0, q2, o2, 0.0f, NULL) == SF_OK);
  EXPECT(sf_attend(two, 0, 0, q2, o2, 0.0f, NULL) == SF_E_ARG);
  EXPECT(sf_attend(two, SF_MAX_BATCH + 1, 0, q2, o2, 0.0f, NULL) == SF_E_ARG);
  /* a corrupted state is refused, not read past its end */
  memset(st, 0xA5, sb);
  EXPECT(sf_state_import(b2, st, sb) != SF_OK);
  free(st);
  /* tracing is refused on dry handles */
  EXPECT(sf_profile_enable(b, 1) == SF_E_STATE);
  sf_kernel_times kt;
  EXPECT(sf_kernel_times_read(b, &kt) == SF_OK);
  EXPECT(sf_buffer_destroy(b2) == SF_OK);
  EXPECT(sf_buffer_destroy(b) == SF_OK);
}

int main(void) {
  /* the served rollout's shape, and smaller ones with every option */
  sf_config served = make(24 * 42, 96, 2, 24, 16, 64, 28, SF_BF16, 5, SF_ROPE_CALLER, 0);
  run_sequence(&served, 40, 1);
  sf_config small = make(12, 4, 2, 8, 2, 64, 3, SF_BF16, 0, SF_ROPE_CALLER, 0);
  run_sequence(&small, 30, 0);
  sf_config sink = make(9, 3, 1, 5, 2, 128, 2, SF_F32, 2, SF_ROPE_CALLER, 0);
  run_sequence(&sink, 25, 0);
  sf_config rope = make(10, 5, 3, 9, 4, 64, 2, SF_BF16, 3, SF_ROPE_LEVEL_REPLACE, 1);
  run_sequence(&rope, 22, 0);
  sf_config rope_add = make(10, 5, 3, 9, 4, 128, 1, SF_BF16, 0, SF_ROPE_LEVEL_ADD, 1);
  run_sequence(&rope_add, 22, 1);
  sf_config long_h = make(45 * 80, 256, 4, 96, 24, 128, 2, SF_BF16, 0, SF_ROPE_CALLER, 0);
  run_sequence(&long_h, 110, 1);

  /* invalid configs and NULL arguments */
  sf_config bad = small;
  bad.w = bad.y;
  EXPECT(sf_config_check(&bad) == SF_E_ARG && sf_buffer_bytes(&bad) == 0);
  bad = small;
  bad.head_dim = 96;
  EXPECT(sf_config_check(&bad) != SF_OK);
  bad = small;
  bad.sink_gap = 1;
  EXPECT(sf_config_check(&bad) != SF_OK);
  EXPECT(sf_config_check(NULL) == SF_E_ARG);
  sf_buffer* nb = NULL;
  EXPECT(sf_buffer_create(&small, NULL, 16, NULL, &nb) != SF_OK && nb == NULL);
  EXPECT(sf_buffer_create(NULL, NULL, 0, NULL, &nb) == SF_E_ARG);
  EXPECT(sf_buffer_destroy(NULL) == SF_OK);
  EXPECT(sf_write_record(NULL, 0, 0, NULL, NULL, NULL) == SF_E_ARG);
  EXPECT(sf_query(NULL, NULL) == SF_E_ARG);
  EXPECT(sf_last_error(NULL) != NULL);
  for (int s = 0; s >= -6; --s) EXPECT(sf_status_str((sf_status)s) != NULL);
  EXPECT(sf_status_str((sf_status)-99) != NULL);
  /* the calibration copy's argument checks (no launch) */
  EXPECT(sf_debug_lds_copy((void*)0x100000, (const void*)0x200000, 0, NULL) == SF_OK);
  EXPECT(sf_debug_lds_copy(NULL, (const void*)0x200000, 16384, NULL) == SF_E_ARG);
  EXPECT(sf_debug_lds_copy((void*)0x100008, (const void*)0x200000, 16384, NULL) == SF_E_ARG);
  EXPECT(sf_debug_lds_copy((void*)0x100000, (const void*)0x102000, 16384, NULL) == SF_E_ARG);
  printf("host API checks passed\n");
  return failures;
}
