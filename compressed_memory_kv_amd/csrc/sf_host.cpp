// Host side of the C-ABI: config checks, the slot map and fill state of each
// session, ordering rules, and kernel enqueue.  No device memory is ever
// allocated here; every pointer comes from the caller.
//
// Model card "GTA world model: weights and inference code":
//   "A frame is a record"       record(t) = H*W raw rows then X summary rows.
//   "What a frame attends to"   frame t sees itself, the Y frames before it
//                               whole, older frames inside the window W as
//                               summaries, and frame 0 whole.
//   "One buffer, no mask"       Z0 | RAW (Y+1 records) | SUM ((W-Y) x X rows);
//                               the figure "The buffer one frame apart" fixes
//                               the rotation (frame 31 takes frame 28's RAW
//                               place, frame 28's summary takes frame 6's SUM
//                               place), read here as RAW slot t mod (Y+1) and
//                               SUM slot f mod (W-Y) for the summarised frame f.
//   "The rest of the model"     the clean pass rewrites the frame's entry.
//   "Running for a long time"   the streaming sink: Z0's keys turned forward after
//                               an eviction step once the gap reaches sink_gap.
//   "Telling a summary from a pixel: level planes"
//                               the temporal band and the level planes applied at
//                               the write and to the query; the construction check.
//   "Files", "Credits"          the optional recency bias on summary keys, by age.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "sf_internal.h"

namespace {

thread_local std::string g_thread_error;
}  // namespace

namespace sf {
LaunchEvents& launch_events() {
  thread_local LaunchEvents ev = {nullptr, nullptr, 0};
  return ev;
}
}  // namespace sf

namespace {

constexpr int64_t kMaxRowsPerBuffer = (int64_t)1 << 30;
constexpr int64_t kMaxElemsPerBlockTensor = (int64_t)1 << 31;

int64_t elem_bytes(int32_t dtype) { return dtype == SF_BF16 ? 2 : 4; }

// Device tensors of a call are read and written in 16-byte vectors.
bool aligned16(const void* a, const void* b = nullptr) {
  return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0;
}

struct Geo {
  int64_t R, C, row_elems, tensor_bytes, block_stride, kv_bytes, scratch_off, scratch_bytes, qrot_off;
  int64_t bias_tab_off, bias_tab_bytes, bias_row_off, total;
};

// Dims of the temporal band of a head (Wan2.1 split: hd - 4*floor(hd/6), first in the head).
int temporal_dims(int head_dim) { return head_dim - 4 * (head_dim / 6); }

// [level] The construction check: both level planes (the two slowest temporal planes) turn
// by less than half a radian over 1024 frames, so they carry no usable position.
bool level_planes_idle(const sf_config& c) {
  const int dim_t = temporal_dims(c.head_dim);
  const int slow = dim_t / 2 - 2;  // the faster of the two
  return std::pow((double)c.rope_theta, -2.0 * slow / dim_t) * 1024.0 < 0.5;
}

sf_status check_config(const sf_config* c, std::string* why) {
  if (!c) { *why = "config is NULL"; return SF_E_ARG; }
  if (c->hw < 1 || c->x < 1 || c->y < 0 || c->w <= c->y || c->n_heads < 1 || c->n_blocks < 1 ||
      c->max_frames < 0) {
    *why = "config needs hw >= 1, x >= 1, y >= 0, w > y, n_heads >= 1, n_blocks >= 1, max_frames >= 0";
    return SF_E_ARG;
  }
  if (c->dtype != SF_F32 && c->dtype != SF_BF16) { *why = "dtype must be SF_F32 or SF_BF16"; return SF_E_ARG; }
  if (c->recency_bias != 0 && c->recency_bias != 1) { *why = "recency_bias must be 0 or 1"; return SF_E_ARG; }
  if (c->rope_mode != SF_ROPE_CALLER && c->rope_mode != SF_ROPE_LEVEL_REPLACE && c->rope_mode != SF_ROPE_LEVEL_ADD) {
    *why = "rope_mode must be SF_ROPE_CALLER, SF_ROPE_LEVEL_REPLACE or SF_ROPE_LEVEL_ADD";
    return SF_E_ARG;
  }
  if (c->sink_gap < 0 || c->sink_gap == 1 || ((c->sink_gap > 0 || c->rope_mode != SF_ROPE_CALLER) &&
                                              !(c->rope_theta > 1.0f))) {
    *why = "sink_gap must be 0 (off) or >= 2, and rope_theta > 1 when the sink or the rope mode uses it";
    return SF_E_ARG;
  }
  if (c->head_dim != 64 && c->head_dim != 128) { *why = "head_dim must be 64 or 128"; return SF_E_UNSUPPORTED; }
  if (c->rope_mode != SF_ROPE_CALLER && !level_planes_idle(*c)) {
    *why = "the two slowest temporal planes turn by 0.5 rad or more over 1024 frames at this rope_theta: "
           "they are not idle and cannot carry the level axis";
    return SF_E_UNSUPPORTED;
  }
  if (c->y + 1 > 4096 || c->w - c->y > (1 << 20) || c->n_blocks > 4096 || c->n_heads > 4096) {
    *why = "config too large (y+1 <= 4096, w-y <= 2^20, n_blocks <= 4096, n_heads <= 4096)";
    return SF_E_UNSUPPORTED;
  }
  const int64_t R = (int64_t)c->hw + c->x;
  const int64_t C = R * (c->y + 2) + (int64_t)(c->w - c->y) * c->x;
  // Kernels address one block's K or V (and q, out) with 32-bit element offsets.
  if (R > (1 << 24) || C > kMaxRowsPerBuffer || C * c->n_heads * (int64_t)c->head_dim >= kMaxElemsPerBlockTensor) {
    *why = "a block's K or V must hold fewer than 2^31 elements";
    return SF_E_UNSUPPORTED;
  }
  return SF_OK;
}

Geo geometry(const sf_config* c) {
  Geo g;
  g.R = (int64_t)c->hw + c->x;
  g.C = g.R * (c->y + 2) + (int64_t)(c->w - c->y) * c->x;
  g.row_elems = (int64_t)c->n_heads * c->head_dim;
  g.tensor_bytes = g.C * g.row_elems * elem_bytes(c->dtype);
  g.block_stride = 2 * g.tensor_bytes;
  g.kv_bytes = g.block_stride * c->n_blocks;
  g.scratch_off = (g.kv_bytes + 255) / 256 * 256;
  // bf16 head_dim 64 reads through the stream-K kernel, or the split-key kernel with a recency bias
  g.scratch_bytes = c->dtype != SF_BF16 ? 0
                    : c->head_dim == 64 && !c->recency_bias
                        ? (int64_t)sf::sk_scratch_bytes(g.R, c->n_heads, g.C)
                        : (int64_t)sf::attend_scratch_bytes(g.R, c->n_heads, c->head_dim);
  auto align256 = [](int64_t x) { return (x + 255) / 256 * 256; };
  int64_t end = g.scratch_off + g.scratch_bytes;
  // a rotated query (rope modes): R rows, 256-byte aligned after the scratch
  g.qrot_off = align256(end);
  if (c->rope_mode != SF_ROPE_CALLER) end = g.qrot_off + g.R * g.row_elems * elem_bytes(c->dtype);
  // recency bias: the table [H][W+1] (zero-filled at create, padded to 256 bytes), then
  // the per-row biases of the current frame [H][C], fp32
  g.bias_tab_off = align256(end);
  g.bias_tab_bytes = c->recency_bias ? align256((int64_t)c->n_heads * (c->w + 1) * 4) : 0;
  g.bias_row_off = g.bias_tab_off + g.bias_tab_bytes;
  if (c->recency_bias) end = g.bias_row_off + (int64_t)c->n_heads * g.C * 4;
  g.total = end;
  return g;
}

// Slot map and fill state of one session.
struct Slots {
  int64_t t_cur = -1;
  int64_t evicted_for = -1;
  int64_t z0_frame = 0;            // frame id Z0's keys are rotated to ([sink])
  std::vector<int64_t> raw_frame;  // frame in each RAW slot, -1 empty
  std::vector<int64_t> sum_frame;  // frame summarised in each SUM slot, -1 empty
};

// [sink] The shift T by which Z0's keys turn after an eviction step: when the oldest
// generated frame in memory is sink_gap or more frames past Z0's frame id, back to a
// gap of 1.  0: nothing to do.
int64_t sink_shift(const sf_config& c, const Slots& s) {
  if (c.sink_gap <= 0) return 0;
  int64_t oldest = -1;
  for (int64_t f : s.raw_frame)
    if (f >= 1 && (oldest < 0 || f < oldest)) oldest = f;
  for (int64_t f : s.sum_frame)
    if (f >= 1 && (oldest < 0 || f < oldest)) oldest = f;
  if (oldest < 0 || oldest - s.z0_frame < c.sink_gap) return 0;
  return oldest - 1 - s.z0_frame;
}

// [sink], [level] Temporal planes of a head in the rotary table and their cosines and
// sines for a turn of T frames (fp64, stored as fp32).
sf::SinkTable rope_table(const sf_config& c, int64_t T) {
  sf::SinkTable tab;
  std::memset(&tab, 0, sizeof(tab));
  const int dim_t = temporal_dims(c.head_dim);
  tab.n_planes = dim_t / 2;
  for (int i = 0; i < tab.n_planes; ++i) {
    const double omega = std::pow((double)c.rope_theta, -2.0 * i / dim_t);
    const double a = omega * (double)T;
    tab.c[i] = (float)std::cos(a);
    tab.s[i] = (float)std::sin(a);
  }
  return tab;
}

struct Segs {
  int n = 0;
  int64_t begin[SF_MAX_SEGMENTS] = {0, 0, 0, 0};
  int64_t len[SF_MAX_SEGMENTS] = {0, 0, 0, 0};
  int64_t keys = 0;
};

// Filled rows as ascending contiguous segments: Z0, occupied RAW slots,
// occupied SUM slots, merged where they touch.
bool readable(const sf_config& c, const Geo& g, const Slots& s, Segs* out) {
  Segs r;
  if (s.t_cur < 0) { *out = r; return true; }
  auto add = [&](int64_t lo, int64_t hi) -> bool {
    if (r.n > 0 && r.begin[r.n - 1] + r.len[r.n - 1] == lo) {
      r.len[r.n - 1] += hi - lo;
    } else {
      if (r.n == SF_MAX_SEGMENTS) return false;
      r.begin[r.n] = lo;
      r.len[r.n] = hi - lo;
      ++r.n;
    }
    r.keys += hi - lo;
    return true;
  };
  if (!add(0, g.R)) return false;
  for (int sl = 0; sl <= c.y; ++sl)
    if (s.raw_frame[sl] >= 1 && !add(g.R * (1 + sl), g.R * (2 + sl))) return false;
  const int64_t base = g.R * (c.y + 2);
  for (int u = 0; u < c.w - c.y; ++u)
    if (s.sum_frame[u] >= 1 && !add(base + (int64_t)u * c.x, base + (int64_t)(u + 1) * c.x)) return false;
  *out = r;
  return true;
}

}  // namespace

// Event pairs bracketing each launch while tracing is on.
struct Tracer {
  bool on = false;
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> pending;  // (kind, (start, end))
  std::vector<hipEvent_t> free_events;
  hipEvent_t get() {
    if (!free_events.empty()) {
      hipEvent_t e = free_events.back();
      free_events.pop_back();
      return e;
    }
    // Device-scope release: the event does not wait for a system-wide flush,
    // so the pair brackets the kernel more tightly.
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventReleaseToDevice) != hipSuccess) return nullptr;
    return e;
  }
  void clear() {
    for (auto& p : pending) {
      free_events.push_back(p.second.first);
      free_events.push_back(p.second.second);
    }
    pending.clear();
  }
  ~Tracer() {
    clear();
    for (hipEvent_t e : free_events) (void)hipEventDestroy(e);
  }
};

struct sf_buffer {
  sf_config cfg;
  Geo geo;
  char* mem = nullptr;
  bool dry = false;
  Slots slots;
  std::vector<int64_t> written_at;  // per block: newest frame written, -1 none
  bool fail_next = false;
  std::string err;
  Tracer trace;
  int64_t bias_t = -1;  // frame whose per-row recency biases the device holds; -1: none
};

namespace {

// Times one launch when tracing is on.  By default the launch stamps the two events
// itself (the dispatch's own start and end); `record_around` records them on the stream
// around the enclosed launches instead (for a call that makes several).
struct TraceScope {
  Tracer& t;
  int kind;
  hipStream_t st;
  bool around;
  hipEvent_t a = nullptr, b = nullptr;
  TraceScope(Tracer& tr, int k, hipStream_t s, bool record_around = false)
      : t(tr), kind(k), st(s), around(record_around) {
    if (!t.on) return;
    a = t.get();
    b = t.get();
    if (a && b) {
      if (!around) {
        sf::launch_events() = {a, b, 0};
        return;
      }
      if (hipEventRecord(a, st) == hipSuccess) return;
    }
    if (a) t.free_events.push_back(a);
    if (b) t.free_events.push_back(b);
    a = b = nullptr;
  }
  ~TraceScope() {
    if (!t.on || !a || !b) return;
    bool ok;
    if (around) {
      ok = hipEventRecord(b, st) == hipSuccess;
    } else {
      sf::LaunchEvents& ev = sf::launch_events();
      ok = ev.launched == 1;  // exactly one dispatch stamped both events
      ev = {nullptr, nullptr, 0};
    }
    if (ok) {
      t.pending.push_back({kind, {a, b}});
    } else {
      t.free_events.push_back(a);
      t.free_events.push_back(b);
    }
  }
};

}  // namespace

namespace {

sf_status fail(sf_buffer* b, sf_status s, const std::string& msg) {
  g_thread_error = msg;
  if (b) b->err = msg;
  return s;
}

sf_status hip_fail(sf_buffer* b, hipError_t e, const char* what) {
  return fail(b, SF_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool all_written(const sf_buffer* b, int64_t t) {
  for (int64_t w : b->written_at)
    if (w != t) return false;
  return true;
}

// Test hook check: consumes the injected failure.
bool take_injected(sf_buffer* b) {
  if (!b->fail_next) return false;
  b->fail_next = false;
  return true;
}

// ---- eviction ------------------------------------------------------------
struct EvictPlan {
  bool copy = false;
  int s = -1;
  int u = -1;
  int64_t f = -1;
};

sf_status check_evict(sf_buffer* b, int64_t t, EvictPlan* plan, bool* noop) {
  const sf_config& c = b->cfg;
  *noop = false;
  if (c.max_frames > 0 && t >= c.max_frames) return fail(b, SF_E_RANGE, "frame id at or beyond max_frames");
  if (t < 0) return fail(b, SF_E_ARG, "negative frame id");
  if (t != b->slots.t_cur + 1) return fail(b, SF_E_ORDER, "sf_evict(t) needs t == t_cur + 1");
  if (b->slots.t_cur >= 0 && !all_written(b, b->slots.t_cur))
    return fail(b, SF_E_ORDER, "sf_evict: some block has not been written at the current frame");
  if (b->slots.evicted_for == t) { *noop = true; return SF_OK; }
  EvictPlan p;
  if (t > c.y) {
    const int s = (int)(t % (c.y + 1));
    const int64_t f = b->slots.raw_frame[s];
    if (f >= 1) {
      p.copy = true;
      p.s = s;
      p.f = f;
      p.u = (int)(f % (c.w - c.y));
    }
  }
  *plan = p;
  return SF_OK;
}

sf_status apply_evict(sf_buffer* b, int64_t t, const EvictPlan& p, hipStream_t st) {
  const sf_config& c = b->cfg;
  if (p.copy && take_injected(b)) return fail(b, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)");
  if (p.copy && !b->dry) {
    const int64_t eb = elem_bytes(c.dtype);
    const int64_t row_bytes = b->geo.row_elems * eb;
    const int64_t src = (b->geo.R * (1 + p.s) + c.hw) * row_bytes;
    const int64_t dst = (b->geo.R * (c.y + 2) + (int64_t)p.u * c.x) * row_bytes;
    TraceScope ts(b->trace, SF_K_EVICT, st);
    hipError_t e = sf::launch_evict(b->mem, c.n_blocks, (size_t)b->geo.block_stride, (size_t)b->geo.tensor_bytes,
                                    (size_t)src, (size_t)dst, (size_t)(c.x * row_bytes), st);
    if (e != hipSuccess) return hip_fail(b, e, "evict launch");
  }
  if (p.copy) b->slots.sum_frame[p.u] = p.f;
  b->slots.evicted_for = t;
  const int64_t T = sink_shift(c, b->slots);
  if (T > 0) {
    if (take_injected(b)) return fail(b, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)");
    if (!b->dry) {
      TraceScope ts(b->trace, SF_K_SINK, st);
      // under the replace reading a summary row's level planes hold no time: kept
      const int lvl_row0 = c.rope_mode == SF_ROPE_LEVEL_REPLACE ? c.hw : (int)b->geo.R;
      hipError_t e = sf::launch_sink_rotate(b->mem, c.n_blocks, (size_t)b->geo.block_stride, lvl_row0,
                                            (int)b->geo.R, c.n_heads, c.head_dim, c.dtype == SF_BF16,
                                            rope_table(c, T), st);
      if (e != hipSuccess) return hip_fail(b, e, "sink rotation launch");
    }
    b->slots.z0_frame += T;
  }
  return SF_OK;
}

// ---- record write ---------------------------------------------------------
sf_status check_write(sf_buffer* b, int32_t block, int64_t t, const void* k, const void* v, bool assume_evicted) {
  const sf_config& c = b->cfg;
  if (block < 0 || block >= c.n_blocks) return fail(b, SF_E_ARG, "block index out of range");
  if (t < 0) return fail(b, SF_E_ARG, "negative frame id");
  if (c.max_frames > 0 && t >= c.max_frames) return fail(b, SF_E_RANGE, "frame id at or beyond max_frames");
  if (!b->dry && (!k || !v)) return fail(b, SF_E_ARG, "k or v is NULL");
  // every kernel that reads a record moves it in 16-byte vectors
  if (!b->dry && !aligned16(k, v)) return fail(b, SF_E_ARG, "k and v must be 16-byte aligned");
  if (t == b->slots.t_cur) return SF_OK;  // rewrite of the current frame (clean pass)
  if (t != b->slots.t_cur + 1) return fail(b, SF_E_ORDER, "sf_write_record(t) needs t == t_cur or t_cur + 1");
  if (b->slots.t_cur >= 0 && !all_written(b, b->slots.t_cur))
    return fail(b, SF_E_ORDER, "advance before every block holds the current frame");
  if (t >= 1) {
    const int s = (int)(t % (c.y + 1));
    const int64_t f = b->slots.raw_frame[s];
    if (f >= 1 && b->slots.evicted_for != t && !assume_evicted)
      return fail(b, SF_E_ORDER, "the frame leaving this RAW slot has not been evicted (call sf_evict first)");
  }
  return SF_OK;
}

// First buffer row of frame t's record: Z0 or its RAW slot.
int64_t record_row0(const sf_buffer* b, int64_t t) {
  return t == 0 ? 0 : b->geo.R * (1 + t % (b->cfg.y + 1));
}

// The slot state after writing frame t's record into block `block`.
void write_state(sf_buffer* b, int32_t block, int64_t t) {
  if (t != b->slots.t_cur) {
    b->slots.t_cur = t;
    if (t >= 1) b->slots.raw_frame[t % (b->cfg.y + 1)] = t;
  }
  b->written_at[block] = t;
}

// The record write.  Under a rope mode, `q` (if not NULL) is turned in the same launch
// into the session's query rows (sf_step: the query belongs to the frame just written).
sf_status launch_write(sf_buffer* b, int32_t block, int64_t t, const void* k, const void* v, hipStream_t st,
                       const void* q = nullptr) {
  const int64_t row_bytes = b->geo.row_elems * elem_bytes(b->cfg.dtype);
  char* kb = b->mem + block * b->geo.block_stride + record_row0(b, t) * row_bytes;
  char* vb = kb + b->geo.tensor_bytes;
  const sf_config& c = b->cfg;
  TraceScope ts(b->trace, SF_K_WRITE, st);
  hipError_t e;
  if (c.rope_mode == SF_ROPE_CALLER) {
    e = sf::launch_copy_rows(kb, vb, k, v, (size_t)(b->geo.R * row_bytes), st);
  } else {
    const sf::RopeJob job = {kb, vb, q ? b->mem + b->geo.qrot_off : nullptr, k, v, q};
    e = sf::launch_rope_rows(job, (int)b->geo.R, c.hw, c.n_heads, c.head_dim, c.dtype == SF_BF16, c.rope_mode,
                             rope_table(c, t), st);
  }
  if (e != hipSuccess) return hip_fail(b, e, "write launch");
  return SF_OK;
}

sf_status apply_write(sf_buffer* b, int32_t block, int64_t t, const void* k, const void* v, hipStream_t st) {
  if (take_injected(b)) return fail(b, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)");
  if (!b->dry) {
    sf_status s = launch_write(b, block, t, k, v, st);
    if (s != SF_OK) return s;
  }
  write_state(b, block, t);
  return SF_OK;
}

// ---- attention -------------------------------------------------------------
sf_status check_attend_one(sf_buffer* b, int32_t block, bool after_write) {
  if (block < 0 || block >= b->cfg.n_blocks) return fail(b, SF_E_ARG, "block index out of range");
  if (!after_write && (b->slots.t_cur < 0 || b->written_at[block] != b->slots.t_cur))
    return fail(b, SF_E_STATE, "sf_attend: the block does not hold the current frame");
  // Once the next frame's eviction step has run, the memory no longer holds what frame
  // t_cur sees ([attends]): the leaving frame's summary has replaced an older one in SUM,
  // and the sink may have turned Z0; the read waits for the next frame's write.
  if (!after_write && b->slots.evicted_for == b->slots.t_cur + 1)
    return fail(b, SF_E_STATE, "sf_attend: the next frame's eviction has run; write frame t_cur + 1 first");
  return SF_OK;
}

// Device scratch a read takes from one region instead of the sessions' own memory: the
// partial results of split reads and the turned queries of rope modes, laid out one after
// the other (256-byte aligned).  NULL: every session uses its own scratch region.
// A planning arena (plan = true) only adds up the bytes: the reads it is passed to lay
// out their scratch and launch nothing.
struct Arena {
  char* base;
  size_t cap;
  size_t used;
  bool plan;
  char* take(size_t bytes) {
    const size_t need = (bytes + 255) / 256 * 256;
    if (need > cap - used) return nullptr;
    char* p = base + used;
    used += need;
    return p;
  }
};
bool planning(const Arena* a) { return a && a->plan; }

// [level] A query under a rope mode, turned by the session's current frame into the
// session's own memory (or the arena); *qs is then what the read uses.  Other sessions:
// *qs = q.
sf_status stage_query(sf_buffer* b, const void* q, const void** qs, hipStream_t st, Arena* arena = nullptr) {
  *qs = q;
  const sf_config& c = b->cfg;
  if (c.rope_mode == SF_ROPE_CALLER || b->dry) return SF_OK;
  char* dst = b->mem + b->geo.qrot_off;
  if (arena) {
    dst = arena->take((size_t)(b->geo.R * b->geo.row_elems * elem_bytes(c.dtype)));
    if (!dst) return fail(b, SF_E_UNSUPPORTED, "sf_attend_static_scratch: the static scratch array is too small");
    if (arena->plan) return SF_OK;
  }
  TraceScope ts(b->trace, SF_K_ROPE, st);
  const sf::RopeJob job = {nullptr, nullptr, dst, nullptr, nullptr, q};
  hipError_t e = sf::launch_rope_rows(job, (int)b->geo.R, c.hw, c.n_heads, c.head_dim, c.dtype == SF_BF16,
                                      c.rope_mode, rope_table(c, b->slots.t_cur), st);
  if (e != hipSuccess) return hip_fail(b, e, "query rotation launch");
  *qs = dst;
  return SF_OK;
}

// [files], [credits] The per-row recency biases for the session's current frame, rebuilt on
// the read's stream when the frame (or the table) changed since the last build.
sf_status refresh_bias(sf_buffer* b, hipStream_t st) {
  const sf_config& c = b->cfg;
  if (!c.recency_bias || b->dry || b->bias_t == b->slots.t_cur) return SF_OK;
  sf::BiasGeo g;
  g.rows = (int32_t)b->geo.R;
  g.hw = c.hw;
  g.x = c.x;
  g.y = c.y;
  g.w = c.w;
  g.heads = c.n_heads;
  g.capacity = (int32_t)b->geo.C;
  g.pad = 0;
  g.t = b->slots.t_cur;
  TraceScope ts(b->trace, SF_K_BIAS, st);
  hipError_t e = sf::launch_bias_rows(reinterpret_cast<float*>(b->mem + b->geo.bias_row_off),
                                      reinterpret_cast<const float*>(b->mem + b->geo.bias_tab_off), g, st);
  if (e != hipSuccess) return hip_fail(b, e, "recency bias launch");
  b->bias_t = b->slots.t_cur;
  return SF_OK;
}

// Compute units of the current device (cached per device).
int device_cu_count() {
  static std::atomic<int> cache[64];  // 0 until asked; every thread that asks stores the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// bf16, head_dim 64: persistent stream-K kernel, then the combine of split units.
// A record that the attention launch writes itself (sf_step, bf16 head_dim 64): source
// tensors and the buffer row it goes to.
struct RecWrite {
  const void* k;
  const void* v;
  int64_t row0;
};

// The readable segments with the record's rows [row0, row0 + rows) cut out as a segment
// of their own whose rows count in the record's source; *rec_seg is its index (-1 if the
// record is not inside one readable segment or the cut needs too many segments).
Segs cut_record(const Segs& sg, int64_t row0, int64_t rows, int* rec_seg) {
  // The buffer's readable rows without the record's, in slots 0.., and the record in
  // slot kRecSlot.  Keys are summed in any order, so the record's keys go last.
  Segs o;
  *rec_seg = -1;
  o.keys = sg.keys;
  bool found = false;
  auto add = [&](int64_t b, int64_t l) {
    if (l <= 0) return true;
    if (o.n >= sf::kRecSlot) return false;
    o.begin[o.n] = b;
    o.len[o.n] = l;
    ++o.n;
    return true;
  };
  for (int j = 0; j < sg.n; ++j) {
    const int64_t b0 = sg.begin[j], e0 = b0 + sg.len[j];
    if (!found && row0 >= b0 && row0 + rows <= e0) {
      found = true;
      if (!add(b0, row0 - b0) || !add(row0 + rows, e0 - row0 - rows)) return sg;
    } else if (!add(b0, sg.len[j])) {
      return sg;
    }
  }
  if (!found) return sg;
  o.begin[sf::kRecSlot] = 0;
  o.len[sf::kRecSlot] = rows;
  *rec_seg = sf::kRecSlot;
  return o;
}

// sf_debug_range_form: 0 the library's choice, 1 the kernel's formula (32-bit where it
// fits), 2 the kernel's formula in 64-bit arithmetic.
std::atomic<int> g_range_form{0};

sf_status enqueue_attend_sk(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q,
                            void* const* out, float scale_log2, hipStream_t st, const RecWrite* rec = nullptr,
                            Arena* arena = nullptr) {
  sf_buffer* b0 = bufs[0];
  const int H = b0->cfg.n_heads;
  for (int first = 0; first < n; first += sf::kMaxLaunchSessions) {
    const int cnt = n - first < sf::kMaxLaunchSessions ? n - first : sf::kMaxLaunchSessions;
    sf::SkLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.n_sessions = cnt;
    a.n_heads = H;
    a.scale_log2 = scale_log2;
    int64_t iters = 0, units_total = 0, cost = 0;
    const int piece_cost = sf::kSkPieceCost;
    bool any_tail = false;
    int64_t qmax = 1;
    for (int i = 0; i < cnt; ++i) {
      sf_buffer* b = bufs[first + i];
      Segs sg;
      readable(b->cfg, b->geo, b->slots, &sg);
      sf::SkSession& s = a.s[i];
      s.rec_seg = -1;
      if (rec && n == 1) {
        int rs = -1;
        Segs cut = cut_record(sg, rec->row0, b->geo.R, &rs);
        if (rs < 0) return fail(b0, SF_E_STATE, "sf_step: record rows are not readable");
        sg = cut;
        s.rec_seg = rs;
        s.rec_k = rec->k;
        s.rec_v = rec->v;
        s.rec_row0 = (int32_t)rec->row0;
      }
      s.q = q[first + i];
      s.out = static_cast<float*>(out[first + i]);
      s.k = b->mem + block * b->geo.block_stride;
      s.v = b->mem + block * b->geo.block_stride + b->geo.tensor_bytes;
      s.rows = (int32_t)b->geo.R;
      s.n_keys = (int32_t)sg.keys;
      s.n_seg = sg.n;
      for (int j = 0; j < SF_MAX_SEGMENTS; ++j) {
        s.seg_begin[j] = (int32_t)sg.begin[j];
        s.seg_len[j] = (int32_t)sg.len[j];
      }
      s.qtiles = (int32_t)((b->geo.R + sf::kSkRows - 1) / sf::kSkRows);
      s.ntiles = (int32_t)(sg.keys / sf::kSkKeys);
      any_tail = any_tail || (sg.keys % sf::kSkKeys) != 0;
      units_total += (int64_t)H * s.qtiles;
      qmax = s.qtiles > qmax ? s.qtiles : qmax;
    }
    // Groups of workgroups sharing key ranges, one query tile per member: as many members as
    // the most query tiles of a session, at most one XCD's share of the workgroups, whole
    // groups on each XCD (the hardware deals workgroup g to XCD g mod 8).
    int64_t G = (int64_t)sf::kSkWgPerCu * device_cu_count();
    if (G >= 8) G -= G % 8;
    if (G < 1) G = 1;
    const bool by_xcd = G >= 8 && G % 8 == 0;
    const int64_t per_x = by_xcd ? G / 8 : G;
    const int64_t GS = qmax < per_x ? qmax : per_x;
    int64_t gpx = by_xcd ? per_x / GS : 0;
    int64_t NG = by_xcd ? 8 * gpx : G / GS;
    int64_t mmax = 1;
    for (int i = 0; i < cnt; ++i) {
      sf::SkSession& s = a.s[i];
      s.mult = (int32_t)((s.qtiles + GS - 1) / GS);
      mmax = s.mult > mmax ? s.mult : mmax;
      s.it_begin = (int32_t)iters;
      s.cost_begin = (int32_t)cost;
      iters += (int64_t)H * s.ntiles;
      cost += s.ntiles > 0 ? (int64_t)H * s.mult * (s.ntiles + piece_cost) : 0;
    }
    if (iters >= ((int64_t)1 << 30) || units_total >= ((int64_t)1 << 28) || cost >= ((int64_t)1 << 31))
      return fail(b0, SF_E_UNSUPPORTED, "attention launch too large");
    // Every group range spans at least mmax * kSkMinRange cost units (so at least
    // kSkMinRange tiles of any column it starts inside); with fewer, fewer groups, laid out
    // in order.
    if (NG > cost / (sf::kSkMinRange * mmax)) {
      NG = cost / (sf::kSkMinRange * mmax);
      if (NG < 1) NG = 1;
      gpx = 0;
      G = NG * GS;
    }
    a.n_wg = (int32_t)G;
    a.n_grp = (int32_t)NG;
    a.grp_size = (int32_t)GS;
    a.grp_per_xcd = (int32_t)gpx;
    a.n_iters = (int32_t)iters;
    a.piece_cost = piece_cost;
    a.total_cost = (int32_t)cost;
    const int form = g_range_form.load(std::memory_order_relaxed);
    a.narrow = (cost + 1) * NG < ((int64_t)1 << 31) && form != 2 ? 1 : 0;
    // the record copy goes to the attention launch's workgroups past the whole groups, if any
    a.rec_copy_idle = cnt == 1 && a.s[0].rec_seg >= 0 && iters > 0 && gpx > 0 && per_x > gpx * GS ? 1 : 0;
    // First column iteration at or past cost C: the first tile whose cost, mult *
    // (piece_cost + t) from its column's start, is at least C.
    auto iter_at_cost = [&](int64_t C) -> int64_t {
      if (C >= cost) return iters;
      int si = 0;
      for (int i = 0; i < cnt; ++i)
        if (a.s[i].ntiles > 0 && a.s[i].cost_begin <= C) si = i;
      const sf::SkSession& s = a.s[si];
      const int64_t m = s.mult, per = m * (s.ntiles + piece_cost), r0 = C - s.cost_begin;
      const int64_t col = r0 / per;
      const int64_t t = (r0 - col * per + m - 1) / m - piece_cost;
      return s.it_begin + col * s.ntiles + (t > 0 ? t : 0);
    };
    // Group g takes the iterations [gstart[g], gstart[g+1]).  The kernel's own formula cuts
    // at costs floor(g*T/NG); the host table may cut at costs weighted per group instead:
    // of the two workgroups a CU holds, the one dispatched first issues faster (measured
    // 0.98 against 1.09 us per tile at the served shape), and the remap puts whole groups on
    // one side, so groups of first-dispatched workgroups get more cost units.
    std::vector<int64_t> gstart((size_t)NG + 1);
    auto cut = [&](bool weighted) {
      std::vector<double> w((size_t)NG, 1.0);
      if (weighted) {
        for (int64_t g = 0; g < NG; ++g) {
          double sum = 0.0;
          for (int64_t j = 0; j < GS; ++j) {
            const int64_t lw = (g % gpx) * GS + j;  // logical workgroup within the XCD
            sum += lw < per_x / 2 ? 1.0 + sf::kSkDispatchSkew / 2 : 1.0 - sf::kSkDispatchSkew / 2;
          }
          w[(size_t)g] = sum / (double)GS;
        }
      }
      double total = 0.0;
      for (double x : w) total += x;
      double acc = 0.0;
      for (int64_t g = 0; g < NG; ++g) {
        const int64_t C = weighted ? (int64_t)((double)cost * (acc / total)) : g * cost / NG;
        gstart[(size_t)g] = iter_at_cost(C);
        acc += w[(size_t)g];
      }
      gstart[(size_t)NG] = iters;
    };
    // Group holding iteration i: the last g whose range starts at or before it.
    auto grp_at = [&](int64_t i) -> int64_t {
      return (int64_t)(std::upper_bound(gstart.begin(), gstart.begin() + NG, i) - gstart.begin()) - 1;
    };
    // Partial-result slots per unit: the groups its column meets, then one for the tail.
    // With the formula's cut a group range holds at least kSkMinRange tiles of a column it
    // starts inside, so this never exceeds the capacity bound the session's own scratch
    // region is sized for; a weighted cut that would is dropped for the formula's.
    auto slots_fit = [&]() {
      for (int i = 0; i < cnt; ++i) {
        sf::SkSession& s = a.s[i];
        int64_t pieces = 0;
        for (int64_t h = 0; s.ntiles > 0 && h < H; ++h) {
          const int64_t c0 = s.it_begin + h * s.ntiles;
          const int64_t p = grp_at(c0 + s.ntiles - 1) - grp_at(c0) + 1;
          pieces = p > pieces ? p : pieces;
        }
        s.ppu = (int32_t)(pieces + 1);
        if (s.ppu > sf::sk_pieces_per_unit(bufs[first + i]->geo.C)) return false;
      }
      return true;
    };
    const bool table = NG <= sf::kSkGrpTable && iters < ((int64_t)1 << 24) && iters > 0 && form == 0;
    // (single-session launches only: the 8-session batched read measured 183.9 us unweighted
    // against 189.7 weighted, the served read 40.7 against 39.5)
    const bool skew = table && cnt == 1 && gpx > 0 && G == (int64_t)sf::kSkWgPerCu * device_cu_count() && sf::kSkWgPerCu == 2;
    cut(skew);
    bool fit = slots_fit();
    if (!fit && skew) {
      cut(false);
      fit = slots_fit();
    }
    if (!fit) return fail(b0, SF_E_UNSUPPORTED, "internal: stream-K partial slots exceed the session's scratch bound");
    // Group starts and first-piece slots, tabulated (see SkLaunch::grp_table).  Without the
    // table the kernel computes the formula's cut itself, which gstart then equals.
    a.grp_table = 0;
    if (table) {
      bool fits = true;
      for (int64_t g = 0; g <= NG && fits; ++g) {
        const int64_t it = gstart[(size_t)g];
        int64_t k = 0;
        if (g < NG && it < iters) {
          int si = 0;
          for (int i = 0; i < cnt; ++i)
            if (a.s[i].it_begin <= it) si = i;
          const sf::SkSession& s = a.s[si];
          const int64_t c0 = s.it_begin + (it - s.it_begin) / s.ntiles * s.ntiles;
          k = g - grp_at(c0);
        }
        fits = k >= 0 && k < 128;
        a.grp_first[g] = (int32_t)(it | (k << 24));
      }
      a.grp_table = fits ? 1 : 0;
      if (!fits && skew) {
        cut(false);  // the kernel computes the formula's cut
        if (!slots_fit()) return fail(b0, SF_E_UNSUPPORTED, "internal: stream-K partial slots exceed the session's scratch bound");
      }
    }
    for (int i = 0; i < cnt; ++i) {
      sf_buffer* b = bufs[first + i];
      sf::SkSession& s = a.s[i];
      const int64_t units = (int64_t)H * s.qtiles;
      const size_t bytes = (size_t)units * s.ppu * sf::kSkRows * (64 + 2) * sizeof(float);
      char* base = b->mem + b->geo.scratch_off;
      if (arena) {
        base = arena->take(bytes);
        if (!base)
          return fail(b0, SF_E_UNSUPPORTED, "sf_attend_static_scratch: the read needs more scratch than the static "
                                            "array holds (" + std::to_string(SF_STATIC_SCRATCH_BYTES) + " bytes)");
      }
      s.part_o = reinterpret_cast<float*>(base);
      s.part_ml = s.part_o + (size_t)units * s.ppu * sf::kSkRows * 64;
    }
    a.uni_units = H * a.s[0].qtiles;
    for (int i = 1; i < cnt; ++i)
      if (a.s[i].qtiles != a.s[0].qtiles) a.uni_units = 0;
    // Producing XCD of every unit (with whole groups per XCD, group g is on XCD
    // g / grp_per_xcd): the XCD of the group holding its column's first tile; a unit
    // without full tiles goes with the unit before it.
    a.xcd_map = 0;
    if (gpx > 0 && iters > 0) {
      int64_t count[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      int x_prev = 0;
      for (int i = 0; i < cnt; ++i) {
        const sf::SkSession& s = a.s[i];
        const int64_t units = (int64_t)H * s.qtiles;
        for (int64_t u = 0; u < units; ++u) {
          int x = x_prev;
          if (s.ntiles > 0) x = (int)(grp_at(s.it_begin + u / s.qtiles * s.ntiles) / gpx);
          x = x < x_prev ? x_prev : (x > 7 ? 7 : x);
          x_prev = x;
          ++count[x];
        }
      }
      a.xcd_first[0] = 0;
      int64_t per = 0;
      for (int x = 0; x < 8; ++x) {
        a.xcd_first[x + 1] = a.xcd_first[x] + (int32_t)count[x];
        per = count[x] > per ? count[x] : per;
      }
      a.xcd_per = (int32_t)per;
      // only when the XCDs hold about the same number of units: otherwise the busiest one
      // would serialize the tail and combine launches
      const int64_t mean = (units_total + 7) / 8;
      a.xcd_map = 4 * per <= 5 * mean ? 1 : 0;
    }
    // the tails ride on the attention launch when it runs (see SkLaunch::tail_units)
    a.tail_units = any_tail && iters > 0 ? (int32_t)units_total : 0;
    if (planning(arena)) continue;
    hipError_t e = hipSuccess;
    if (iters > 0) {
      TraceScope ts(b0->trace, SF_K_ATTEND, st);
      e = sf::launch_attend_sk(a, st);
    }
    if (e != hipSuccess) return hip_fail(b0, e, "attention launch");
    if (any_tail && iters == 0) {
      TraceScope ts(b0->trace, SF_K_TAIL, st);
      e = sf::launch_tail_sk(a, (int)units_total, st);
    }
    if (e != hipSuccess) return hip_fail(b0, e, "attention tail launch");
    {
      TraceScope ts(b0->trace, SF_K_COMBINE, st);
      e = sf::launch_combine_sk(a, (int)units_total, st);
    }
    if (e != hipSuccess) return hip_fail(b0, e, "combine launch");
  }
  return SF_OK;
}

// The split-key (bf16) or fp32 read; sessions with a recency bias get their per-row biases.
sf_status enqueue_attend_split(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q,
                               void* const* out, float scale_log2, hipStream_t st, Arena* arena = nullptr) {
  sf_buffer* b0 = bufs[0];
  const sf_config& c0 = b0->cfg;
  for (int first = 0; first < n; first += sf::kMaxLaunchSessions) {
    const int cnt = n - first < sf::kMaxLaunchSessions ? n - first : sf::kMaxLaunchSessions;
    sf::AttnLaunch a;
    std::memset(&a, 0, sizeof(a));
    a.n_sessions = cnt;
    a.n_heads = c0.n_heads;
    a.head_dim = c0.head_dim;
    a.scale_log2 = scale_log2;
    const bool bf16 = c0.dtype == SF_BF16;
    const int rows_per_tile = bf16 ? sf::kBf16RowsPerTile : sf::kF32RowsPerTile;
    // Key split.  When the (session, head, query tile) units fit in one round of resident
    // workgroups, the split s minimises rounds(s) * ceil(tiles / s) + s (the last term for the
    // combine's reads); otherwise aim at about four workgroups per compute unit.
    int64_t base_units = 0, total_tiles = 0, max_tiles = 0;
    bool launch_bias = false;
    std::vector<Segs> segs(cnt);
    for (int i = 0; i < cnt; ++i) {
      sf_buffer* b = bufs[first + i];
      readable(b->cfg, b->geo, b->slots, &segs[i]);
      const int64_t qt = (b->geo.R + rows_per_tile - 1) / rows_per_tile;
      const int64_t tiles = (segs[i].keys + sf::kBf16KeysPerTile - 1) / sf::kBf16KeysPerTile;
      base_units += qt * c0.n_heads;
      total_tiles += qt * c0.n_heads * tiles;
      max_tiles = tiles > max_tiles ? tiles : max_tiles;
      launch_bias = launch_bias || b->cfg.recency_bias;
    }
    const int64_t target_units = 1024;
    int64_t tiles_per_unit = (total_tiles + target_units - 1) / target_units;
    if (tiles_per_unit < 4) tiles_per_unit = 4;
    int64_t round_split = 0;
    if (bf16 && base_units > 0) {
      const int64_t slots = (int64_t)device_cu_count() * sf::attend_bf16_wgs_per_cu(c0.head_dim, launch_bias);
      if (base_units <= slots) {
        int64_t best = -1;
        for (int64_t sp = 1; sp <= sf::kMaxSplit && sp <= (max_tiles > 0 ? max_tiles : 1); ++sp) {
          const int64_t cost = (base_units * sp + slots - 1) / slots * ((max_tiles + sp - 1) / sp) + sp;
          if (best < 0 || cost < best) {
            best = cost;
            round_split = sp;
          }
        }
      }
    }
    // SF_ATTN_SPLIT=n forces n key splits per (session, head, query tile) (tuning only:
    // results change only by rounding).
    static const int forced_split = [] {
      const char* e = std::getenv("SF_ATTN_SPLIT");
      return e ? std::atoi(e) : 0;
    }();
    int64_t units = 0;
    bool any_bias = false;
    for (int i = 0; i < cnt; ++i) {
      sf_buffer* b = bufs[first + i];
      sf::AttnSession& s = a.s[i];
      if (b->cfg.recency_bias) {
        sf_status r = planning(arena) ? SF_OK : refresh_bias(b, st);
        if (r != SF_OK) return fail(b0, r, b->err);
        s.bias = reinterpret_cast<const float*>(b->mem + b->geo.bias_row_off);
        s.bias_stride = (int32_t)b->geo.C;
        any_bias = true;
      }
      s.q = q[first + i];
      s.out = static_cast<float*>(out[first + i]);
      s.k = b->mem + block * b->geo.block_stride;
      s.v = b->mem + block * b->geo.block_stride + b->geo.tensor_bytes;
      s.part_o = reinterpret_cast<float*>(b->mem + b->geo.scratch_off);
      s.part_ml = s.part_o + (size_t)sf::kMaxSplit * b->geo.R * c0.n_heads * c0.head_dim;
      s.rows = (int32_t)b->geo.R;
      s.n_keys = (int32_t)segs[i].keys;
      s.n_seg = segs[i].n;
      for (int j = 0; j < segs[i].n; ++j) {
        s.seg_begin[j] = (int32_t)segs[i].begin[j];
        s.seg_len[j] = (int32_t)segs[i].len[j];
      }
      s.qtiles = (int32_t)((b->geo.R + rows_per_tile - 1) / rows_per_tile);
      int64_t split = 1;
      if (bf16) {
        const int64_t tiles = (segs[i].keys + sf::kBf16KeysPerTile - 1) / sf::kBf16KeysPerTile;
        split = forced_split > 0 ? forced_split
                : round_split > 0 ? round_split
                                  : (tiles + tiles_per_unit - 1) / tiles_per_unit;
        if (split > sf::kMaxSplit) split = sf::kMaxSplit;
        if (split > tiles) split = tiles;
        if (split < 1) split = 1;
      }
      s.split = (int32_t)split;
      if (arena && split > 1) {
        const size_t slice = (size_t)b->geo.R * c0.n_heads;
        char* base = arena->take((size_t)split * slice * (c0.head_dim + 2) * sizeof(float));
        if (!base)
          return fail(b0, SF_E_UNSUPPORTED, "sf_attend_static_scratch: the read needs more scratch than the static "
                                            "array holds (" + std::to_string(SF_STATIC_SCRATCH_BYTES) + " bytes)");
        s.part_o = reinterpret_cast<float*>(base);
        s.part_ml = s.part_o + (size_t)split * slice * c0.head_dim;
      }
      s.unit_begin = (int32_t)units;
      units += (int64_t)s.qtiles * c0.n_heads * split;
    }
    (void)base_units;
    if (units >= ((int64_t)1 << 30)) return fail(b0, SF_E_UNSUPPORTED, "attention launch too large");
    a.total_units = (int32_t)units;
    if (planning(arena)) continue;
    hipError_t e;
    {
      TraceScope ts(b0->trace, SF_K_ATTEND, st);
      e = bf16 ? sf::launch_attend_bf16(a, any_bias, st) : sf::launch_attend_f32(a, any_bias, st);
    }
    if (e != hipSuccess) return hip_fail(b0, e, "attention launch");
    if (bf16) {
      TraceScope ts(b0->trace, SF_K_COMBINE, st);
      e = sf::launch_combine(a, st);
      if (e != hipSuccess) return hip_fail(b0, e, "combine launch");
    }
  }
  return SF_OK;
}

sf_status enqueue_attend(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q, void* const* out,
                         float scale, hipStream_t st, Arena* arena = nullptr) {
  const sf_config& c0 = bufs[0]->cfg;
  const float sc = scale > 0.0f ? scale : 1.0f / std::sqrt((float)c0.head_dim);
  const float scale_log2 = sc * 1.4426950408889634f;
  if (c0.dtype != SF_BF16 || c0.head_dim != 64)
    return enqueue_attend_split(bufs, n, block, q, out, scale_log2, st, arena);
  // bf16 head_dim 64: the stream-K kernel, except for sessions with a recency bias
  sf_buffer* gb[2][SF_MAX_BATCH];
  const void* gq[2][SF_MAX_BATCH];
  void* go[2][SF_MAX_BATCH];
  int cnt[2] = {0, 0};
  for (int i = 0; i < n; ++i) {
    const int k = bufs[i]->cfg.recency_bias ? 1 : 0;
    gb[k][cnt[k]] = bufs[i];
    gq[k][cnt[k]] = q[i];
    go[k][cnt[k]] = out[i];
    ++cnt[k];
  }
  if (cnt[0] > 0) {
    sf_status s = enqueue_attend_sk(gb[0], cnt[0], block, gq[0], go[0], scale_log2, st, nullptr, arena);
    if (s != SF_OK) return s;
  }
  if (cnt[1] == 0) return SF_OK;
  return enqueue_attend_split(gb[1], cnt[1], block, gq[1], go[1], scale_log2, st, arena);
}

void fill_view(const sf_config& c, const Geo& g, const Slots& s, int32_t blocks_written, sf_view* v) {
  Segs r;
  readable(c, g, s, &r);
  v->t_cur = s.t_cur;
  v->n_keys = r.keys;
  v->evicted_for = s.evicted_for;
  v->n_seg = r.n;
  v->raw_slot = s.t_cur >= 1 ? (int32_t)(s.t_cur % (c.y + 1)) : -1;
  v->blocks_written = blocks_written;
  v->reserved = 0;
  for (int i = 0; i < SF_MAX_SEGMENTS; ++i) {
    v->seg_begin[i] = i < r.n ? r.begin[i] : 0;
    v->seg_len[i] = i < r.n ? r.len[i] : 0;
  }
  if (v->raw_frame)
    for (int i = 0; i <= c.y; ++i) v->raw_frame[i] = s.raw_frame[i];
  if (v->sum_frame)
    for (int i = 0; i < c.w - c.y; ++i) v->sum_frame[i] = s.sum_frame[i];
  v->z0_frame = s.z0_frame;
}

}  // namespace

extern "C" {

sf_status sf_config_check(const sf_config* cfg) {
  std::string why;
  sf_status s = check_config(cfg, &why);
  if (s != SF_OK) g_thread_error = why;
  return s;
}

size_t sf_buffer_bytes(const sf_config* cfg) {
  std::string why;
  if (check_config(cfg, &why) != SF_OK) return 0;
  return (size_t)geometry(cfg).total;
}

size_t sf_kv_bytes(const sf_config* cfg) {
  std::string why;
  if (check_config(cfg, &why) != SF_OK) return 0;
  return (size_t)geometry(cfg).kv_bytes;
}

int64_t sf_kv_offset(const sf_config* cfg, int32_t block, int32_t which) {
  std::string why;
  if (check_config(cfg, &why) != SF_OK || block < 0 || block >= cfg->n_blocks || (which != 0 && which != 1))
    return -1;
  const Geo g = geometry(cfg);
  return block * g.block_stride + which * g.tensor_bytes;
}

sf_status sf_buffer_create(const sf_config* cfg, void* dev_mem, size_t bytes, void* hip_stream, sf_buffer** out) {
  std::string why;
  if (!out) return fail(nullptr, SF_E_ARG, "out is NULL");
  *out = nullptr;
  sf_status st = check_config(cfg, &why);
  if (st != SF_OK) return fail(nullptr, st, why);
  const Geo g = geometry(cfg);
  const bool dry = dev_mem == nullptr && bytes == 0;
  if (!dry) {
    if (!dev_mem) return fail(nullptr, SF_E_ARG, "dev_mem is NULL but bytes > 0");
    if (bytes < (size_t)g.total) return fail(nullptr, SF_E_ARG, "device memory smaller than sf_buffer_bytes(cfg)");
    if (reinterpret_cast<uintptr_t>(dev_mem) & 15u) return fail(nullptr, SF_E_ARG, "device memory not 16-byte aligned");
  }
  sf_buffer* b = new (std::nothrow) sf_buffer();
  if (!b) return fail(nullptr, SF_E_ARG, "out of host memory");
  b->cfg = *cfg;
  b->geo = g;
  b->mem = static_cast<char*>(dev_mem);
  b->dry = dry;
  b->slots.raw_frame.assign(cfg->y + 1, -1);
  b->slots.sum_frame.assign(cfg->w - cfg->y, -1);
  b->written_at.assign(cfg->n_blocks, -1);
  if (!dry) {
    hipError_t e = sf::launch_fill_zero(dev_mem, (size_t)g.kv_bytes, static_cast<hipStream_t>(hip_stream));
    if (e == hipSuccess && g.bias_tab_bytes > 0)
      e = sf::launch_fill_zero(static_cast<char*>(dev_mem) + g.bias_tab_off, (size_t)g.bias_tab_bytes,
                               static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) {
      delete b;
      return fail(nullptr, SF_E_HIP, std::string("zero fill launch: ") + hipGetErrorString(e));
    }
  }
  *out = b;
  return SF_OK;
}

sf_status sf_buffer_destroy(sf_buffer* buf) {
  delete buf;
  return SF_OK;
}

sf_status sf_write_record(sf_buffer* buf, int32_t block, int64_t t, const void* k, const void* v, void* hip_stream) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  sf_status s = check_write(buf, block, t, k, v, false);
  if (s != SF_OK) return s;
  return apply_write(buf, block, t, k, v, static_cast<hipStream_t>(hip_stream));
}

sf_status sf_record_slot(sf_buffer* buf, int32_t block, int64_t t, void** k_rows, void** v_rows) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  if (!k_rows || !v_rows) return fail(buf, SF_E_ARG, "sf_record_slot: k_rows or v_rows is NULL");
  if (buf->cfg.rope_mode != SF_ROPE_CALLER)
    return fail(buf, SF_E_UNSUPPORTED, "sf_record_slot: rows are stored as given; not under a rope mode");
  // the same checks as a write; the pointers stand in for the caller's data
  alignas(16) static const char stand_in[16] = {};
  sf_status s = check_write(buf, block, t, stand_in, stand_in, false);
  if (s != SF_OK) return s;
  if (buf->dry) {
    *k_rows = *v_rows = nullptr;
    return SF_OK;
  }
  const int64_t row_bytes = buf->geo.row_elems * elem_bytes(buf->cfg.dtype);
  char* kb = buf->mem + block * buf->geo.block_stride + record_row0(buf, t) * row_bytes;
  *k_rows = kb;
  *v_rows = kb + buf->geo.tensor_bytes;
  return SF_OK;
}

sf_status sf_commit_record(sf_buffer* buf, int32_t block, int64_t t) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  if (buf->cfg.rope_mode != SF_ROPE_CALLER)
    return fail(buf, SF_E_UNSUPPORTED, "sf_commit_record: rows are stored as given; not under a rope mode");
  alignas(16) static const char stand_in[16] = {};
  sf_status s = check_write(buf, block, t, stand_in, stand_in, false);
  if (s != SF_OK) return s;
  write_state(buf, block, t);
  return SF_OK;
}

// Host state layout: magic, version, the config, then int64 t_cur, evicted_for, z0_frame,
// raw_frame[y+1], sum_frame[w-y], written_at[n_blocks].
static const uint32_t kStateMagic = 0x31534653u;  // "SFS1"

size_t sf_state_bytes(const sf_config* cfg) {
  std::string why;
  if (check_config(cfg, &why) != SF_OK) return 0;
  return 8 + sizeof(sf_config) + 8 * (3 + (size_t)(cfg->y + 1) + (size_t)(cfg->w - cfg->y) + (size_t)cfg->n_blocks);
}

sf_status sf_state_export(const sf_buffer* buf, void* dst, size_t bytes) {
  if (!buf || !dst) return fail(nullptr, SF_E_ARG, "sf_state_export: NULL argument");
  const size_t need = sf_state_bytes(&buf->cfg);
  if (bytes < need) return fail(nullptr, SF_E_ARG, "sf_state_export: destination smaller than sf_state_bytes");
  char* p = static_cast<char*>(dst);
  const uint32_t head[2] = {kStateMagic, 1u};
  std::memcpy(p, head, 8);
  p += 8;
  std::memcpy(p, &buf->cfg, sizeof(sf_config));
  p += sizeof(sf_config);
  auto put = [&](int64_t x) { std::memcpy(p, &x, 8); p += 8; };
  put(buf->slots.t_cur);
  put(buf->slots.evicted_for);
  put(buf->slots.z0_frame);
  for (int64_t f : buf->slots.raw_frame) put(f);
  for (int64_t f : buf->slots.sum_frame) put(f);
  for (int64_t f : buf->written_at) put(f);
  return SF_OK;
}

sf_status sf_state_import(sf_buffer* buf, const void* src, size_t bytes) {
  if (!buf || !src) return fail(nullptr, SF_E_ARG, "sf_state_import: NULL argument");
  const sf_config& c = buf->cfg;
  if (bytes < sf_state_bytes(&c)) return fail(buf, SF_E_ARG, "sf_state_import: fewer bytes than sf_state_bytes");
  const char* p = static_cast<const char*>(src);
  uint32_t head[2];
  std::memcpy(head, p, 8);
  p += 8;
  if (head[0] != kStateMagic || head[1] != 1u) return fail(buf, SF_E_ARG, "sf_state_import: not a state record");
  if (std::memcmp(p, &c, sizeof(sf_config)) != 0)
    return fail(buf, SF_E_ARG, "sf_state_import: the state belongs to another config");
  p += sizeof(sf_config);
  auto get = [&]() { int64_t x; std::memcpy(&x, p, 8); p += 8; return x; };
  Slots s;
  s.t_cur = get();
  s.evicted_for = get();
  s.z0_frame = get();
  s.raw_frame.resize(c.y + 1);
  s.sum_frame.resize(c.w - c.y);
  for (auto& f : s.raw_frame) f = get();
  for (auto& f : s.sum_frame) f = get();
  std::vector<int64_t> wa(c.n_blocks);
  for (auto& f : wa) f = get();
  // consistency: every slot holds a frame it can hold at t_cur
  bool ok = s.t_cur >= -1 && (c.max_frames == 0 || s.t_cur < c.max_frames) && s.evicted_for <= s.t_cur + 1 &&
            s.z0_frame >= 0 && s.z0_frame <= (s.t_cur > 0 ? s.t_cur : 0);
  for (int i = 0; i <= c.y && ok; ++i) {
    const int64_t f = s.raw_frame[i];
    ok = f == -1 || (f >= 1 && f <= s.t_cur && f % (c.y + 1) == i && f > s.t_cur - (c.y + 1));
  }
  for (int u = 0; u < c.w - c.y && ok; ++u) {
    const int64_t f = s.sum_frame[u];
    ok = f == -1 || (f >= 1 && f % (c.w - c.y) == u && f <= s.t_cur - (c.y + 1) + (s.evicted_for > s.t_cur));
  }
  for (int64_t f : wa) ok = ok && f >= -1 && f <= s.t_cur && (s.t_cur < 0 || f >= s.t_cur - 1);
  if (!ok) return fail(buf, SF_E_ARG, "sf_state_import: inconsistent state");
  buf->slots = s;
  buf->written_at = wa;
  buf->bias_t = -1;
  return SF_OK;
}

sf_status sf_evict(sf_buffer* buf, int64_t t, void* hip_stream) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  EvictPlan p;
  bool noop = false;
  sf_status s = check_evict(buf, t, &p, &noop);
  if (s != SF_OK || noop) return s;
  return apply_evict(buf, t, p, static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"

namespace {

// The library's own device scratch for sf_attend_static_scratch: one array per device that
// holds the library, reached through the address hipGetSymbolAddress gives for the device
// (the array's name in host code is a host-side stand-in, not a device address).
static __device__ __align__(256) char scratch[SF_STATIC_SCRATCH_BYTES];

// Address of the current device's copy of the array, looked up once per device.
sf_status static_scratch(char** out) {
  static std::atomic<char*> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, SF_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(nullptr, SF_E_UNSUPPORTED, "sf_attend_static_scratch: device index >= 64");
  char* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !addr)
      return fail(nullptr, SF_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    p = static_cast<char*>(addr);
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SF_OK;
}

// sf_attend; with static_scratch_arena, the read's scratch comes from this device's copy of
// the static array instead of the sessions' memory.
sf_status attend_impl(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q, void* const* out,
                      float scale, void* hip_stream, bool static_scratch_arena) {
  if (!bufs || n < 1 || n > SF_MAX_BATCH) return fail(nullptr, SF_E_ARG, "sf_attend: need 1 <= n <= SF_MAX_BATCH");
  if (!bufs[0]) return fail(nullptr, SF_E_ARG, "sf_attend: NULL buffer");
  const sf_config& c0 = bufs[0]->cfg;
  const bool dry = bufs[0]->dry;
  if (!dry && (!q || !out)) return fail(bufs[0], SF_E_ARG, "sf_attend: q or out array is NULL");
  if (!(scale == scale) || std::isinf(scale)) return fail(bufs[0], SF_E_ARG, "sf_attend: scale is not finite");
  for (int i = 0; i < n; ++i) {
    sf_buffer* b = bufs[i];
    if (!b) return fail(bufs[0], SF_E_ARG, "sf_attend: NULL buffer");
    if (b->dry != dry) return fail(bufs[0], SF_E_ARG, "sf_attend: dry-run and real buffers mixed");
    if (b->cfg.n_heads != c0.n_heads || b->cfg.head_dim != c0.head_dim || b->cfg.dtype != c0.dtype)
      return fail(bufs[0], SF_E_ARG, "sf_attend: sessions differ in n_heads, head_dim or dtype");
    for (int j = 0; j < i; ++j)
      if (bufs[j] == b) return fail(bufs[0], SF_E_ARG, "sf_attend: a session is listed twice");
    sf_status s = check_attend_one(b, block, false);
    if (s != SF_OK) return fail(bufs[0], s, b->err);
    if (!dry && (!q[i] || !out[i])) return fail(bufs[0], SF_E_ARG, "sf_attend: q or out pointer is NULL");
    if (!dry && !aligned16(q[i], out[i])) return fail(bufs[0], SF_E_ARG, "sf_attend: q and out must be 16-byte aligned");
  }
  for (int i = 0; i < n; ++i)
    if (take_injected(bufs[i])) return fail(bufs[0], SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)");
  if (dry) return SF_OK;
  Arena arena = {nullptr, SF_STATIC_SCRATCH_BYTES, 0, false};
  Arena* ap = nullptr;
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const void* qs[SF_MAX_BATCH];
  if (static_scratch_arena) {
    // Lay the whole read's scratch out first, so a read that does not fit enqueues nothing.
    Arena plan = {reinterpret_cast<char*>(static_cast<uintptr_t>(256)), SIZE_MAX / 2, 0, true};
    for (int i = 0; i < n; ++i) {
      sf_status s = stage_query(bufs[i], q[i], &qs[i], st, &plan);
      if (s != SF_OK) return fail(bufs[0], s, bufs[i]->err);
    }
    sf_status s = enqueue_attend(bufs, n, block, qs, out, scale, st, &plan);
    if (s != SF_OK) return s;
    if (plan.used > SF_STATIC_SCRATCH_BYTES)
      return fail(bufs[0], SF_E_UNSUPPORTED, "sf_attend_static_scratch: the read needs " + std::to_string(plan.used) +
                                                 " bytes of scratch; the static array holds " +
                                                 std::to_string(SF_STATIC_SCRATCH_BYTES));
    s = static_scratch(&arena.base);
    if (s != SF_OK) return fail(bufs[0], s, g_thread_error);
    ap = &arena;
  }
  for (int i = 0; i < n; ++i) {
    sf_status s = stage_query(bufs[i], q[i], &qs[i], st, ap);
    if (s != SF_OK) return fail(bufs[0], s, bufs[i]->err);
  }
  return enqueue_attend(bufs, n, block, qs, out, scale, st, ap);
}

}  // namespace

extern "C" {

sf_status sf_attend(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q, void* const* out,
                    float scale, void* hip_stream) {
  return attend_impl(bufs, n, block, q, out, scale, hip_stream, false);
}

sf_status sf_attend_static_scratch(sf_buffer* const* bufs, int32_t n, int32_t block, const void* const* q,
                                   void* const* out, float scale, void* hip_stream) {
  return attend_impl(bufs, n, block, q, out, scale, hip_stream, true);
}

sf_status sf_step(sf_buffer* buf, int32_t block, int64_t t, const void* q, const void* k, const void* v, void* out,
                  float scale, void* hip_stream) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (!buf->dry && (!q || !out)) return fail(buf, SF_E_ARG, "sf_step: q or out is NULL");
  if (!buf->dry && !aligned16(q, out)) return fail(buf, SF_E_ARG, "sf_step: q and out must be 16-byte aligned");
  if (!(scale == scale) || std::isinf(scale)) return fail(buf, SF_E_ARG, "sf_step: scale is not finite");
  // Validate every part before enqueueing anything.
  EvictPlan ep;
  bool evict_due = false, noop = true;
  if (t == buf->slots.t_cur + 1 && t >= 1) {
    sf_status s = check_evict(buf, t, &ep, &noop);
    if (s != SF_OK) return s;
    evict_due = !noop;
  }
  sf_status s = check_write(buf, block, t, k, v, evict_due);
  if (s != SF_OK) return s;
  s = check_attend_one(buf, block, true);
  if (s != SF_OK) return s;
  if (t == buf->slots.t_cur && buf->slots.evicted_for == t + 1)
    return fail(buf, SF_E_STATE, "sf_step: rewrite of t_cur after the next frame's eviction; its read would be wrong");
  const Slots saved = buf->slots;
  const std::vector<int64_t> saved_written = buf->written_at;
  auto restore = [&](sf_status r) {
    buf->slots = saved;
    buf->written_at = saved_written;
    buf->bias_t = -1;  // the device may hold the biases of the frame this call advanced to
    return r;
  };
  if (evict_due) {
    s = apply_evict(buf, t, ep, st);
    if (s != SF_OK) return restore(s);
  }
  sf_buffer* one[1] = {buf};
  const void* qs[1] = {q};
  void* outs[1] = {out};
  // bf16, head_dim 64: the attention launch writes the record itself (and reads its keys
  // from k and v) whenever the block has a full 64-key tile after the write and the rows
  // around the record fit the remaining segment slots.  Not under a rope mode (there the
  // stored keys are the turned ones, written first), nor with a recency bias (that read
  // goes through the split-key kernel).
  if (!buf->dry && buf->cfg.dtype == SF_BF16 && buf->cfg.head_dim == 64 && buf->cfg.rope_mode == SF_ROPE_CALLER &&
      !buf->cfg.recency_bias) {
    write_state(buf, block, t);
    Segs sg;
    readable(buf->cfg, buf->geo, buf->slots, &sg);
    int rs = -1;
    cut_record(sg, record_row0(buf, t), buf->geo.R, &rs);
    if (sg.keys >= sf::kSkKeys && rs >= 0) {
      if (take_injected(buf)) return restore(fail(buf, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)"));
      const float sc = scale > 0.0f ? scale : 1.0f / std::sqrt((float)buf->cfg.head_dim);
      const RecWrite rw = {k, v, record_row0(buf, t)};
      s = enqueue_attend_sk(one, 1, block, qs, outs, sc * 1.4426950408889634f, st, &rw);
      if (s != SF_OK) return restore(s);
      return SF_OK;
    }
    if (take_injected(buf)) return restore(fail(buf, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)"));
    s = launch_write(buf, block, t, k, v, st);
    if (s != SF_OK) return restore(s);
  } else if (!buf->dry && buf->cfg.rope_mode != SF_ROPE_CALLER) {
    // the frame's query is turned in the write's launch
    if (take_injected(buf)) return restore(fail(buf, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)"));
    write_state(buf, block, t);
    s = launch_write(buf, block, t, k, v, st, q);
    if (s != SF_OK) return restore(s);
    qs[0] = buf->mem + buf->geo.qrot_off;
  } else {
    s = apply_write(buf, block, t, k, v, st);
    if (s != SF_OK) return restore(s);
  }
  if (take_injected(buf)) return restore(fail(buf, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)"));
  if (buf->dry) return SF_OK;
  s = enqueue_attend(one, 1, block, qs, outs, scale, st);
  if (s != SF_OK) return restore(s);
  return SF_OK;
}

sf_status sf_set_recency_bias(sf_buffer* buf, const float* table, void* hip_stream) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  const sf_config& c = buf->cfg;
  if (!c.recency_bias) return fail(buf, SF_E_UNSUPPORTED, "sf_set_recency_bias: the config has recency_bias = 0");
  if (!buf->dry && (!table || (reinterpret_cast<uintptr_t>(table) & 3u)))
    return fail(buf, SF_E_ARG, "sf_set_recency_bias: table is NULL or not 4-byte aligned");
  if (take_injected(buf)) return fail(buf, SF_E_HIP, "injected launch failure (sf_debug_fail_next_launch)");
  if (buf->dry) return SF_OK;
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  TraceScope ts(buf->trace, SF_K_BIAS, st);
  hipError_t e = sf::launch_bias_table(reinterpret_cast<float*>(buf->mem + buf->geo.bias_tab_off), table,
                                       c.n_heads * (c.w + 1), st);
  if (e != hipSuccess) return hip_fail(buf, e, "recency bias table launch");
  buf->bias_t = -1;
  return SF_OK;
}

sf_status sf_rope_rows(const sf_config* cfg, int64_t t, const void* src, void* dst, void* hip_stream) {
  std::string why;
  sf_status st = check_config(cfg, &why);
  if (st != SF_OK) return fail(nullptr, st, why);
  if (cfg->rope_mode == SF_ROPE_CALLER) return fail(nullptr, SF_E_ARG, "sf_rope_rows: the config's rope mode turns nothing");
  if (t < 0 || (cfg->max_frames > 0 && t >= cfg->max_frames)) return fail(nullptr, SF_E_RANGE, "sf_rope_rows: bad frame id");
  if (!src || !dst) return fail(nullptr, SF_E_ARG, "sf_rope_rows: NULL pointer");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u)
    return fail(nullptr, SF_E_ARG, "sf_rope_rows: pointers must be 16-byte aligned");
  const Geo g = geometry(cfg);
  const sf::RopeJob job = {nullptr, nullptr, dst, nullptr, nullptr, src};
  hipError_t e = sf::launch_rope_rows(job, (int)g.R, cfg->hw, cfg->n_heads, cfg->head_dim, cfg->dtype == SF_BF16,
                                      cfg->rope_mode, rope_table(*cfg, t), static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(nullptr, SF_E_HIP, std::string("sf_rope_rows launch: ") + hipGetErrorString(e));
  return SF_OK;
}

sf_status sf_query(const sf_buffer* buf, sf_view* view) {
  if (!buf || !view) return fail(nullptr, SF_E_ARG, "sf_query: NULL argument");
  int32_t nw = 0;
  for (int64_t w : buf->written_at) nw += (buf->slots.t_cur >= 0 && w == buf->slots.t_cur);
  fill_view(buf->cfg, buf->geo, buf->slots, nw, view);
  return SF_OK;
}

sf_status sf_plan(const sf_config* cfg, int64_t t, sf_view* view) {
  std::string why;
  if (!view) return fail(nullptr, SF_E_ARG, "sf_plan: view is NULL");
  sf_status st = check_config(cfg, &why);
  if (st != SF_OK) return fail(nullptr, st, why);
  if (t < -1) return fail(nullptr, SF_E_ARG, "sf_plan: t < -1");
  if (cfg->max_frames > 0 && t >= cfg->max_frames) return fail(nullptr, SF_E_RANGE, "frame id at or beyond max_frames");
  if (t > ((int64_t)1 << 32)) return fail(nullptr, SF_E_UNSUPPORTED, "sf_plan: t too large");
  const Geo g = geometry(cfg);
  Slots s;
  s.raw_frame.assign(cfg->y + 1, -1);
  s.sum_frame.assign(cfg->w - cfg->y, -1);
  for (int64_t f = 0; f <= t; ++f) {
    if (f > cfg->y) {
      const int sl = (int)(f % (cfg->y + 1));
      const int64_t leaving = s.raw_frame[sl];
      if (leaving >= 1) s.sum_frame[leaving % (cfg->w - cfg->y)] = leaving;
    }
    if (f >= 1) s.z0_frame += sink_shift(*cfg, s);
    if (f >= 1) s.raw_frame[f % (cfg->y + 1)] = f;
    if (f >= 1) s.evicted_for = f;
    s.t_cur = f;
  }
  fill_view(*cfg, g, s, t >= 0 ? cfg->n_blocks : 0, view);
  return SF_OK;
}

const char* sf_status_str(sf_status s) {
  // C callers may pass any int: read the argument's bytes as one (a C++ load of an enum
  // value outside the enumerators' range is undefined).
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case SF_OK: return "SF_OK";
    case SF_E_ARG: return "SF_E_ARG";
    case SF_E_ORDER: return "SF_E_ORDER";
    case SF_E_RANGE: return "SF_E_RANGE";
    case SF_E_STATE: return "SF_E_STATE";
    case SF_E_HIP: return "SF_E_HIP";
    case SF_E_UNSUPPORTED: return "SF_E_UNSUPPORTED";
  }
  return "SF_E_UNKNOWN";
}

const char* sf_last_error(const sf_buffer* buf) { return buf ? buf->err.c_str() : g_thread_error.c_str(); }

sf_status sf_profile_enable(sf_buffer* buf, int32_t on) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  if (buf->dry) return fail(buf, SF_E_STATE, "dry-run handles launch nothing to time");
  if (!on) buf->trace.clear();
  buf->trace.on = on != 0;
  return SF_OK;
}

sf_status sf_kernel_times_read(sf_buffer* buf, sf_kernel_times* out) {
  if (!buf || !out) return fail(buf, SF_E_ARG, "sf_kernel_times_read: NULL argument");
  for (int k = 0; k < SF_K_KINDS; ++k) {
    out->ms[k] = 0.0;
    out->launches[k] = 0;
  }
  for (auto& p : buf->trace.pending) {
    hipError_t e = hipEventSynchronize(p.second.second);
    if (e != hipSuccess) {
      buf->trace.clear();
      return hip_fail(buf, e, "event wait");
    }
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, p.second.first, p.second.second);
    if (e != hipSuccess) {
      buf->trace.clear();
      return hip_fail(buf, e, "event elapsed time");
    }
    out->ms[p.first] += ms;
    out->launches[p.first] += 1;
  }
  buf->trace.clear();
  return SF_OK;
}

sf_status sf_debug_fail_next_launch(sf_buffer* buf) {
  if (!buf) return fail(nullptr, SF_E_ARG, "buffer is NULL");
  buf->fail_next = true;
  return SF_OK;
}

sf_status sf_debug_range_form(int32_t form) {
  if (form < 0 || form > 2) return fail(nullptr, SF_E_ARG, "sf_debug_range_form: form must be 0, 1 or 2");
  g_range_form.store(form, std::memory_order_relaxed);
  return SF_OK;
}

sf_status sf_debug_lds_copy(void* dst, const void* src, size_t bytes, void* hip_stream) {
  if (bytes == 0) return SF_OK;
  if (!dst || !src) return fail(nullptr, SF_E_ARG, "sf_debug_lds_copy: NULL pointer");
  if (!aligned16(dst) || !aligned16(src)) return fail(nullptr, SF_E_ARG, "sf_debug_lds_copy: pointers must be 16-byte aligned");
  if (bytes % 16384 != 0) return fail(nullptr, SF_E_ARG, "sf_debug_lds_copy: bytes must be a multiple of 16384");
  const char* d = static_cast<const char*>(dst);
  const char* s = static_cast<const char*>(src);
  if (d < s + bytes && s < d + bytes) return fail(nullptr, SF_E_ARG, "sf_debug_lds_copy: regions overlap");
  hipError_t e = sf::launch_lds_copy(dst, src, bytes, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(nullptr, SF_E_HIP, std::string("sf_debug_lds_copy: ") + hipGetErrorString(e));
  return SF_OK;
}

}  // extern "C"
