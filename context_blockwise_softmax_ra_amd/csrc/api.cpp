// Host side of libra.so: argument validation, kernel dispatch, the zig-zag
// shard map and the per-rank step plan.  No device allocation, no
// synchronisation; every launch goes on the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <climits>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "ra_internal.h"

namespace {

thread_local std::string g_err;

ra_status fail(ra_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ra_status ok() {
  g_err.clear();
  return RA_OK;
}

}  // namespace

ra_status ra::set_error(ra_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

namespace {

ra_status hip_fail(hipError_t e, const char* what) {
  return fail(RA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int part_len(int full, ra_part p) {
  if (p == RA_PART_ALL) return full;
  const int half = full >> 1;
  return p == RA_PART_FIRST_HALF ? half : full - half;
}

bool bf16_dims_ok(int dqk, int dv) {
  return (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128) || (dqk == 64 && dv == 64);
}
bool f32_dims_ok(int dqk, int dv) {
  return dqk == dv && (dqk == 16 || dqk == 32 || dqk == 64 || dqk == 128);
}

// Validates a cu_seqlens host array: non-negative, non-decreasing.
ra_status check_cu(const int32_t* cu, int n_seq, const char* name) {
  if (!cu) return fail(RA_ERR_INVALID_ARG, "%s is NULL", name);
  if (cu[0] < 0) return fail(RA_ERR_INVALID_ARG, "%s[0] < 0", name);
  for (int s = 0; s < n_seq; ++s)
    if (cu[s + 1] < cu[s]) return fail(RA_ERR_INVALID_ARG, "%s decreases at %d", name, s);
  return RA_OK;
}

struct Checked {
  int64_t qs, ks, vs;
  int total_q, total_k;
  int max_q_part, max_k_part;
  float scale;
};

// Full validation of a block descriptor (q/k/v presence controlled by need_kv).
ra_status check_desc(const ra_attn_desc* d, bool need_kv, Checked* c) {
  if (!d) return fail(RA_ERR_INVALID_ARG, "descriptor is NULL");
  if (!d->q) return fail(RA_ERR_INVALID_ARG, "q is NULL");
  if (need_kv && (!d->k || !d->v)) return fail(RA_ERR_INVALID_ARG, "k or v is NULL");
  if (d->dtype != RA_BF16 && d->dtype != RA_FP32)
    return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", (int)d->dtype);
  if (d->hq <= 0 || d->hkv <= 0) return fail(RA_ERR_INVALID_ARG, "head counts must be > 0");
  if (d->hq % d->hkv)
    return fail(RA_ERR_INVALID_ARG, "hq (%d) is not a multiple of hkv (%d)", d->hq, d->hkv);
  if (d->dqk <= 0 || d->dv <= 0) return fail(RA_ERR_INVALID_ARG, "head dims must be > 0");
  if (d->dtype == RA_BF16 && !bf16_dims_ok(d->dqk, d->dv))
    return fail(RA_ERR_UNSUPPORTED, "bf16 (dqk, dv) = (%d, %d) not built", d->dqk, d->dv);
  if (d->dtype == RA_FP32 && !f32_dims_ok(d->dqk, d->dv))
    return fail(RA_ERR_UNSUPPORTED, "fp32 (dqk, dv) = (%d, %d) not built", d->dqk, d->dv);
  if (d->q_part < RA_PART_ALL || d->q_part > RA_PART_SECOND_HALF || d->k_part < RA_PART_ALL ||
      d->k_part > RA_PART_SECOND_HALF)
    return fail(RA_ERR_INVALID_ARG, "unknown part selector");
  if (d->n_seq <= 0) return fail(RA_ERR_INVALID_ARG, "n_seq must be >= 1");
  if (!d->cu_seqlens_q || !d->cu_seqlens_k)
    return fail(RA_ERR_INVALID_ARG, "device cu_seqlens is NULL");
  ra_status st;
  if ((st = check_cu(d->cu_seqlens_q_host, d->n_seq, "cu_seqlens_q_host")) != RA_OK) return st;
  if ((st = check_cu(d->cu_seqlens_k_host, d->n_seq, "cu_seqlens_k_host")) != RA_OK) return st;
  c->qs = d->q_stride_tok ? d->q_stride_tok : (int64_t)d->hq * d->dqk;
  c->ks = d->k_stride_tok ? d->k_stride_tok : (int64_t)d->hkv * d->dqk;
  c->vs = d->v_stride_tok ? d->v_stride_tok : (int64_t)d->hkv * d->dv;
  if (c->qs < (int64_t)d->hq * d->dqk || c->ks < (int64_t)d->hkv * d->dqk ||
      c->vs < (int64_t)d->hkv * d->dv)
    return fail(RA_ERR_INVALID_ARG, "token stride smaller than heads * dim");
  if (d->dtype == RA_BF16) {
    if (!aligned16(d->q) || (need_kv && (!aligned16(d->k) || !aligned16(d->v))))
      return fail(RA_ERR_INVALID_ARG, "bf16 q/k/v must be 16-byte aligned");
    if ((c->qs % 8) || (c->ks % 8) || (c->vs % 8))
      return fail(RA_ERR_INVALID_ARG, "bf16 token strides must be multiples of 8 elements");
  }
  c->total_q = d->cu_seqlens_q_host[d->n_seq];
  c->total_k = d->cu_seqlens_k_host[d->n_seq];
  c->max_q_part = 0;
  c->max_k_part = 0;
  for (int s = 0; s < d->n_seq; ++s) {
    const int lq = d->cu_seqlens_q_host[s + 1] - d->cu_seqlens_q_host[s];
    const int lk = d->cu_seqlens_k_host[s + 1] - d->cu_seqlens_k_host[s];
    if ((d->q_part != RA_PART_ALL && (lq & 1)) || (d->k_part != RA_PART_ALL && (lk & 1)))
      return fail(RA_ERR_INVALID_ARG, "segment %d: halves need an even length (q %d, k %d)", s,
                  lq, lk);
    const int pq = part_len(lq, d->q_part), pk = part_len(lk, d->k_part);
    if (d->causal && pq != pk)
      return fail(RA_ERR_INVALID_ARG,
                  "segment %d: causal block needs equal q and k part lengths (%d vs %d)", s, pq,
                  pk);
    c->max_q_part = std::max(c->max_q_part, pq);
    c->max_k_part = std::max(c->max_k_part, pk);
  }
  c->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->dqk);
  return RA_OK;
}

ra::AttnArgs make_args(const ra_attn_desc* d, const Checked& c) {
  ra::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = d->q;
  a.k = d->k;
  a.v = d->v;
  a.q_stride = c.qs;
  a.k_stride = c.ks;
  a.v_stride = c.vs;
  a.hq = d->hq;
  a.hkv = d->hkv;
  a.group = d->hq / d->hkv;
  a.n_seq = d->n_seq;
  a.cu_q = d->cu_seqlens_q;
  a.cu_k = d->cu_seqlens_k;
  a.q_part = d->q_part;
  a.k_part = d->k_part;
  const int bm = d->dtype == RA_BF16 ? ra::kFwdBlockM : ra::kF32BlockM;
  a.n_qtiles = (c.max_q_part + bm - 1) / bm;
  a.n_ktiles = 0;
  a.scale = c.scale;
  a.scale_log2 = c.scale * 1.4426950408889634f;
  a.total_q = c.total_q;
  return a;
}

// Which bf16 forward kernel runs a launch.  The 8-wave ping-pong kernel
// works on 256-row query tiles and pays off when its matrix-core phase and
// softmax phase are of similar length and the tiles are well filled: head
// dims 128/128, at least two 256-row tiles (x query heads) per CU of the
// 256, and at least 3/4 of the tiled rows' work being real rows.  Work
// weights each segment's rows by its key count, since short packed
// documents, whose 256-row tiles are mostly padding, carry little of it.
// (128K packed documents split 16 ways: 70% of the tiled rows are real, 82%
// of the work, and the ping-pong kernel is 9% faster there.)  Otherwise the
// 4-wave kernel (128-row tiles) runs.  RA_FWD_KERNEL=pp or =4w in the
// environment forces one.
bool use_pingpong(const ra_attn_desc* d, ra_part q_part) {
  const char* e = std::getenv("RA_FWD_KERNEL");
  if (e && !std::strcmp(e, "pp")) return true;
  if (e && !std::strcmp(e, "4w")) return false;
  if (d->dqk != 128 || d->dv != 128) return false;
  long long tiles = 0;
  double work = 0.0, tiled_work = 0.0;
  for (int s = 0; s < d->n_seq; ++s) {
    const int lq = part_len(d->cu_seqlens_q_host[s + 1] - d->cu_seqlens_q_host[s], q_part);
    const double lk = (double)(d->cu_seqlens_k_host[s + 1] - d->cu_seqlens_k_host[s]);
    const int t = (lq + 255) / 256;
    tiles += t;
    work += (double)lq * lk;
    tiled_work += (double)t * 256.0 * lk;
  }
  return tiles * d->hq >= 2 * 256 && work * 4.0 >= tiled_work * 3.0;
}

ra_status launch_fwd(const ra_attn_desc* d, const Checked& c, float* out, float* lse, bool merge,
                     hipStream_t st) {
  ra::AttnArgs a = make_args(d, c);
  a.out = out;
  a.lse = lse;
  if (a.n_qtiles == 0) return RA_OK;
  hipError_t e;
  if (d->dtype != RA_BF16)
    e = ra::launch_attn_fwd_f32(a, d->dqk, d->dv, d->causal != 0, merge, st);
  else if (use_pingpong(d, d->q_part))
    e = ra::launch_attn_fwd_pp(a, d->dqk, d->dv, d->causal != 0, merge, st);
  else
    e = ra::launch_attn_fwd_bf16(a, d->dqk, d->dv, d->causal != 0, merge, st);
  if (e != hipSuccess) return hip_fail(e, "attention forward launch");
  return RA_OK;
}

ra_status check_merge_args(const float* out_acc, const float* lse_acc, const float* out_part,
                           const float* lse_part, int32_t total_t, int32_t h, int32_t dv,
                           int32_t n_seq, const int32_t* cu, const int32_t* cu_host,
                           ra_part rows, int* max_rows) {
  if (!out_acc || !lse_acc || !out_part || !lse_part || !cu)
    return fail(RA_ERR_INVALID_ARG, "NULL buffer");
  if (total_t < 0 || h <= 0 || dv <= 0 || (dv % 4) || dv > 1024)
    return fail(RA_ERR_INVALID_ARG, "bad sizes (total_t %d, h %d, dv %d)", total_t, h, dv);
  if (!aligned16(out_acc) || !aligned16(out_part))
    return fail(RA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  if (rows < RA_PART_ALL || rows > RA_PART_SECOND_HALF)
    return fail(RA_ERR_INVALID_ARG, "unknown part selector");
  if (n_seq <= 0) return fail(RA_ERR_INVALID_ARG, "n_seq must be >= 1");
  ra_status st = check_cu(cu_host, n_seq, "cu_seqlens_host");
  if (st != RA_OK) return st;
  if (cu_host[n_seq] > total_t) return fail(RA_ERR_INVALID_ARG, "cu_seqlens beyond total_t");
  *max_rows = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int L = cu_host[s + 1] - cu_host[s];
    if (rows != RA_PART_ALL && (L & 1))
      return fail(RA_ERR_INVALID_ARG, "segment %d: halves need an even length", s);
    *max_rows = std::max(*max_rows, part_len(L, rows));
  }
  return RA_OK;
}

// Step s of rank r: owner j = (r - s) mod C (KV moves 0 -> 1 -> ...).
struct Step {
  int owner;
  int causal;
  ra_part q_part, k_part;
};

Step plan_step(int rank, int s, int cp) {
  Step p;
  p.owner = ((rank - s) % cp + cp) % cp;
  int causal, q_part, k_part;
  ra::owner_plan(rank, p.owner, &causal, &q_part, &k_part);
  p.causal = causal;
  p.q_part = (ra_part)q_part;
  p.k_part = (ra_part)k_part;
  return p;
}

ra_status check_rank_common(const ra_attn_desc& L, int cp, int rank, const void* const* kb,
                            const void* const* vb, Checked* c) {
  if (cp <= 0 || rank < 0 || rank >= cp)
    return fail(RA_ERR_INVALID_ARG, "bad cp_size %d / rank %d", cp, rank);
  if (!kb || !vb) return fail(RA_ERR_INVALID_ARG, "k_blocks / v_blocks is NULL");
  for (int j = 0; j < cp; ++j)
    if (!kb[j] || !vb[j]) return fail(RA_ERR_INVALID_ARG, "KV block of owner %d is NULL", j);
  if (L.q_part != RA_PART_ALL || L.k_part != RA_PART_ALL)
    return fail(RA_ERR_INVALID_ARG, "local descriptor parts must be RA_PART_ALL");
  ra_attn_desc t = L;
  t.k = kb[0];
  t.v = vb[0];
  t.causal = 1;
  ra_status st = check_desc(&t, true, c);
  if (st != RA_OK) return st;
  for (int s = 0; s <= L.n_seq; ++s)
    if (L.cu_seqlens_q_host[s] != L.cu_seqlens_k_host[s])
      return fail(RA_ERR_INVALID_ARG, "local q and k cu_seqlens must match");
  // a rank's local buffers start at its first row: the KV-split combine,
  // the cast and delta run over rows [0, cu[n_seq])
  if (L.cu_seqlens_q_host[0] != 0)
    return fail(RA_ERR_INVALID_ARG, "local cu_seqlens must start at 0");
  if (cp > 1)
    for (int s = 0; s < L.n_seq; ++s)
      if ((L.cu_seqlens_q_host[s + 1] - L.cu_seqlens_q_host[s]) & 1)
        return fail(RA_ERR_INVALID_ARG, "local segment %d has odd length (zig-zag halves)", s);
  for (int j = 0; j < cp; ++j)
    if (L.dtype == RA_BF16 && (!aligned16(kb[j]) || !aligned16(vb[j])))
      return fail(RA_ERR_INVALID_ARG, "KV block %d not 16-byte aligned", j);
  return RA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Other shard maps: token lists and the rectangles of one ring step
// ---------------------------------------------------------------------------

// Consecutive global tokens of a rank, at consecutive local rows.
struct Run {
  int64_t local_lo, global_lo, len;
  int doc;
};

ra_status check_map(ra_map kind, int cp, int rank, int n_seq, const int32_t* cu) {
  if (kind < RA_MAP_ZIGZAG || kind > RA_MAP_CONTIGUOUS)
    return fail(RA_ERR_INVALID_ARG, "unknown shard map %d", (int)kind);
  if (cp <= 0 || rank < 0 || rank >= cp)
    return fail(RA_ERR_INVALID_ARG, "bad cp_size %d / rank %d", cp, rank);
  if (n_seq <= 0) return fail(RA_ERR_INVALID_ARG, "n_seq must be >= 1");
  ra_status st = check_cu(cu, n_seq, "cu_seqlens_global");
  if (st != RA_OK) return st;
  if (cu[0] != 0) return fail(RA_ERR_INVALID_ARG, "cu_seqlens_global must start at 0");
  const int64_t T = cu[n_seq];
  if (kind == RA_MAP_ZIGZAG) {
    for (int d = 0; d < n_seq; ++d)
      if ((cu[d + 1] - cu[d]) % (2 * cp))
        return fail(RA_ERR_INVALID_ARG, "sequence %d length is not a multiple of 2*cp_size", d);
  } else if (kind == RA_MAP_ZIGZAG_GLOBAL) {
    if (T % (2 * cp)) return fail(RA_ERR_INVALID_ARG, "stream length not a multiple of 2*cp_size");
  } else if (T % cp) {
    return fail(RA_ERR_INVALID_ARG, "stream length not a multiple of cp_size");
  }
  return RA_OK;
}

// Runs of a rank's tokens (all maps but the striped one), split at document
// boundaries, in local order.
std::vector<Run> rank_runs(ra_map kind, int cp, int r, int n_seq, const int32_t* cu) {
  std::vector<Run> runs;
  const int64_t T = cu[n_seq];
  if (kind == RA_MAP_ZIGZAG) {
    int64_t local = 0;
    for (int d = 0; d < n_seq; ++d) {
      const int64_t c = (cu[d + 1] - cu[d]) / (2 * cp);
      if (c == 0) continue;
      runs.push_back({local, cu[d] + (int64_t)r * c, c, d});
      runs.push_back({local + c, cu[d] + (int64_t)(2 * cp - 1 - r) * c, c, d});
      local += 2 * c;
    }
    return runs;
  }
  std::vector<Run> raw;
  if (kind == RA_MAP_ZIGZAG_GLOBAL) {
    const int64_t c = T / (2 * cp);
    raw.push_back({0, (int64_t)r * c, c, 0});
    raw.push_back({c, (int64_t)(2 * cp - 1 - r) * c, c, 0});
  } else {
    const int64_t L = T / cp;
    raw.push_back({0, (int64_t)r * L, L, 0});
  }
  for (const Run& x : raw) {
    int64_t g = x.global_lo;
    const int64_t end = x.global_lo + x.len;
    int d = (int)(std::upper_bound(cu, cu + n_seq + 1, (int32_t)g) - cu) - 1;
    while (g < end && d < n_seq) {
      const int64_t e = std::min<int64_t>(end, cu[d + 1]);
      if (e > g) runs.push_back({x.local_lo + (g - x.global_lo), g, e - g, d});
      g = std::max<int64_t>(g, e);
      ++d;
    }
  }
  return runs;
}

int64_t ceil_pos(int64_t a, int64_t c) { return a <= 0 ? 0 : (a + c - 1) / c; }

ra_status step_segments(ra_map kind, int cp, int r, int o, int n_seq, const int32_t* cu,
                        std::vector<ra_segment>* out) {
  out->clear();
  auto push = [&](int64_t q_lo, int64_t q_hi, int64_t k_lo, int64_t k_hi, int64_t diag) {
    const int64_t klen = k_hi - k_lo;
    if (q_hi <= q_lo || klen <= 0) return;
    if ((q_hi - q_lo - 1) + diag < 0) return;  // no row sees a key
    if (diag >= klen - 1) diag = klen;         // every key visible
    out->push_back({(int32_t)q_lo, (int32_t)q_hi, (int32_t)k_lo, (int32_t)k_hi, (int32_t)diag});
  };
  if (kind == RA_MAP_STRIPED) {
    // local row i of rank r is token i*cp + r: key j of owner o is not after
    // row i iff j <= i (o <= r) or j <= i - 1 (o > r)
    const int off = o <= r ? 0 : -1;
    for (int d = 0; d < n_seq; ++d) {
      const int64_t qa = ceil_pos(cu[d] - r, cp), qb = ceil_pos(cu[d + 1] - r, cp);
      const int64_t ka = ceil_pos(cu[d] - o, cp), kb = ceil_pos(cu[d + 1] - o, cp);
      push(qa, qb, ka, kb, qa - ka + off);
    }
    return RA_OK;
  }
  const std::vector<Run> qr = rank_runs(kind, cp, r, n_seq, cu);
  const std::vector<Run> kr = rank_runs(kind, cp, o, n_seq, cu);
  std::vector<std::vector<int>> by_doc(n_seq);
  for (int i = 0; i < (int)kr.size(); ++i) by_doc[kr[i].doc].push_back(i);
  for (const Run& p : qr) {
    // key runs of the same document that some row of p can see: all keys
    // before p's first token (full), or overlapping p's range (causal with
    // the offset of their global starts); merged into one rectangle
    int64_t k_lo = -1, k_hi = -1, diag = 0;
    bool full = true;
    for (int i : by_doc[p.doc]) {
      const Run& k = kr[i];
      if (k.global_lo > p.global_lo + p.len - 1) continue;  // after every row
      const bool kfull = k.global_lo + k.len - 1 <= p.global_lo;
      if (k_lo < 0) {
        k_lo = k.local_lo;
      } else if (k.local_lo != k_hi || !full) {
        return fail(RA_ERR_UNSUPPORTED, "step rectangle of rank %d / owner %d not contiguous", r, o);
      }
      if (!kfull) {
        if (p.global_lo - k.global_lo < -1)
          return fail(RA_ERR_UNSUPPORTED, "step rectangle of rank %d / owner %d not expressible", r, o);
        diag = (k.local_lo - k_lo) + (p.global_lo - k.global_lo);
        full = false;
      }
      k_hi = k.local_lo + k.len;
    }
    if (k_lo < 0) continue;
    push(p.local_lo, p.local_lo + p.len, k_lo, k_hi, full ? (k_hi - k_lo) : diag);
  }
  return RA_OK;
}

}  // namespace

extern "C" {

const char* ra_forward_kernel(const ra_attn_desc* d, ra_part q_part) {
  if (!d) {
    fail(RA_ERR_INVALID_ARG, "descriptor is NULL");
    return nullptr;
  }
  if (q_part < RA_PART_ALL || q_part > RA_PART_SECOND_HALF) {
    fail(RA_ERR_INVALID_ARG, "unknown part selector");
    return nullptr;
  }
  if (d->dtype != RA_BF16 && d->dtype != RA_FP32) {
    fail(RA_ERR_INVALID_ARG, "unknown dtype");
    return nullptr;
  }
  if (d->n_seq <= 0 || !d->cu_seqlens_q_host) {
    fail(RA_ERR_INVALID_ARG, "n_seq or cu_seqlens_q_host invalid");
    return nullptr;
  }
  if (check_cu(d->cu_seqlens_q_host, d->n_seq, "cu_seqlens_q_host") != RA_OK) return nullptr;
  if (d->dtype == RA_FP32) return "attn_fwd_f32";
  return use_pingpong(d, q_part) ? "attn_fwd_pp" : "attn_fwd_bf16";
}

const char* ra_last_error(void) { return g_err.c_str(); }

const char* ra_version(void) { return "0.1.0"; }

ra_status ra_block_attn_fwd(const ra_attn_desc* d, float* out, float* lse, void* stream) {
  Checked c;
  ra_status st = check_desc(d, true, &c);
  if (st != RA_OK) return st;
  if (!out || !lse) return fail(RA_ERR_INVALID_ARG, "out or lse is NULL");
  if (!aligned16(out)) return fail(RA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  st = launch_fwd(d, c, out, lse, false, (hipStream_t)stream);
  return st == RA_OK ? ok() : st;
}

ra_status ra_block_attn_fwd_merge(const ra_attn_desc* d, float* out_acc, float* lse_acc,
                                  void* stream) {
  Checked c;
  ra_status st = check_desc(d, true, &c);
  if (st != RA_OK) return st;
  if (!out_acc || !lse_acc) return fail(RA_ERR_INVALID_ARG, "out_acc or lse_acc is NULL");
  if (!aligned16(out_acc)) return fail(RA_ERR_INVALID_ARG, "out_acc must be 16-byte aligned");
  st = launch_fwd(d, c, out_acc, lse_acc, true, (hipStream_t)stream);
  return st == RA_OK ? ok() : st;
}

ra_status ra_lse_merge(float* out_acc, float* lse_acc, const float* out_part,
                       const float* lse_part, int32_t total_t, int32_t h, int32_t dv,
                       int32_t n_seq, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                       ra_part rows, void* stream) {
  int max_rows = 0;
  ra_status st = check_merge_args(out_acc, lse_acc, out_part, lse_part, total_t, h, dv, n_seq,
                                  cu_seqlens, cu_seqlens_host, rows, &max_rows);
  if (st != RA_OK) return st;
  hipError_t e = ra::launch_lse_merge(out_acc, lse_acc, out_part, lse_part, total_t, h, dv,
                                      n_seq, cu_seqlens, rows, max_rows, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "lse merge launch");
  return ok();
}

ra_status ra_zigzag_shard_map(int32_t cp_size, int32_t rank, int32_t n_seq,
                              const int32_t* cu_seqlens_global, int32_t* cu_seqlens_local,
                              int32_t* src_start) {
  if (cp_size <= 0 || rank < 0 || rank >= cp_size)
    return fail(RA_ERR_INVALID_ARG, "bad cp_size %d / rank %d", cp_size, rank);
  if (n_seq <= 0) return fail(RA_ERR_INVALID_ARG, "n_seq must be >= 1");
  if (!cu_seqlens_local || !src_start) return fail(RA_ERR_INVALID_ARG, "NULL output");
  ra_status st = check_cu(cu_seqlens_global, n_seq, "cu_seqlens_global");
  if (st != RA_OK) return st;
  const int two_c = 2 * cp_size;
  for (int s = 0; s < n_seq; ++s) {
    const int L = cu_seqlens_global[s + 1] - cu_seqlens_global[s];
    if (L % two_c)
      return fail(RA_ERR_INVALID_ARG, "sequence %d length %d is not a multiple of 2*cp_size %d",
                  s, L, two_c);
  }
  cu_seqlens_local[0] = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int g0 = cu_seqlens_global[s];
    const int c = (cu_seqlens_global[s + 1] - g0) / two_c;
    src_start[2 * s] = g0 + rank * c;
    src_start[2 * s + 1] = g0 + (two_c - 1 - rank) * c;
    cu_seqlens_local[s + 1] = cu_seqlens_local[s] + 2 * c;
  }
  return ok();
}

static ra_status zigzag_copy(const void* src, void* dst, int64_t row_bytes, int32_t n_seq,
                             const int32_t* cu_local, const int32_t* start,
                             const int32_t* cu_local_host, const int32_t* start_host,
                             int32_t total_global, bool gather, hipStream_t st) {
  if (!src || !dst || !cu_local || !start || !cu_local_host || !start_host)
    return fail(RA_ERR_INVALID_ARG, "NULL argument");
  if (row_bytes <= 0 || (row_bytes % 16) || !aligned16(src) || !aligned16(dst))
    return fail(RA_ERR_INVALID_ARG, "rows must be 16-byte multiples and aligned");
  if (n_seq <= 0) return fail(RA_ERR_INVALID_ARG, "n_seq must be >= 1");
  ra_status s = check_cu(cu_local_host, n_seq, "cu_seqlens_local_host");
  if (s != RA_OK) return s;
  int max_half = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int L = cu_local_host[i + 1] - cu_local_host[i];
    if (L & 1) return fail(RA_ERR_INVALID_ARG, "local segment %d has odd length", i);
    const int c = L / 2;
    for (int j = 0; j < 2; ++j)
      if (start_host[2 * i + j] < 0 || (int64_t)start_host[2 * i + j] + c > total_global)
        return fail(RA_ERR_INVALID_ARG, "segment %d half %d outside the global buffer", i, j);
    max_half = std::max(max_half, c);
  }
  hipError_t e = ra::launch_zigzag_copy(src, dst, row_bytes, n_seq, cu_local, start, max_half,
                                        gather, st);
  if (e != hipSuccess) return hip_fail(e, "zig-zag copy launch");
  return ok();
}

ra_status ra_zigzag_gather(const void* global_src, void* local_dst, int64_t row_bytes,
                           int32_t n_seq, const int32_t* cu_seqlens_local,
                           const int32_t* src_start, const int32_t* cu_seqlens_local_host,
                           const int32_t* src_start_host, int32_t total_global, void* stream) {
  return zigzag_copy(global_src, local_dst, row_bytes, n_seq, cu_seqlens_local, src_start,
                     cu_seqlens_local_host, src_start_host, total_global, true,
                     (hipStream_t)stream);
}

ra_status ra_zigzag_scatter(const void* local_src, void* global_dst, int64_t row_bytes,
                            int32_t n_seq, const int32_t* cu_seqlens_local,
                            const int32_t* src_start, const int32_t* cu_seqlens_local_host,
                            const int32_t* src_start_host, int32_t total_global, void* stream) {
  return zigzag_copy(local_src, global_dst, row_bytes, n_seq, cu_seqlens_local, src_start,
                     cu_seqlens_local_host, src_start_host, total_global, false,
                     (hipStream_t)stream);
}

ra_status ra_cast_f32_bf16(const float* src, void* dst, int64_t n, void* stream) {
  if (!src || !dst) return fail(RA_ERR_INVALID_ARG, "NULL buffer");
  if (n < 0 || (n % 4)) return fail(RA_ERR_INVALID_ARG, "n must be a multiple of 4");
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(dst) & 7u))
    return fail(RA_ERR_INVALID_ARG, "misaligned buffers");
  hipError_t e = ra::launch_cast_f32_bf16(src, dst, n, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cast launch");
  return ok();
}

// KV split of a fused rank share: a launch of the 4-wave kernel with fewer
// than 256 workgroups (a rank share of few rows and heads, or a Ulysses
// share of few heads) leaves CUs idle, so the share's key tiles are dealt
// round-robin over `split` parts (more workgroups), each writing a float32
// partial, and a combine kernel weights the parts by their lse.
// RA_FWD_KV_SPLIT=<n> in the environment forces n parts (1 = none).
constexpr int kMaxFwdSplit = 16;
static int fwd_kv_split(const ra_rank_desc* d, const Checked& c) {
  const ra_attn_desc& L = d->local;
  if (d->fuse_merge != 2 || L.dtype != RA_BF16) return 1;
  if (use_pingpong(&L, RA_PART_ALL)) return 1;
  const char* e = std::getenv("RA_FWD_KV_SPLIT");
  if (e && *e) return std::max(1, std::min(std::atoi(e), kMaxFwdSplit));
  (void)c;
  long long tiles = 0;  // 128-row query tiles of all segments (the launch's grid per head)
  for (int s = 0; s < L.n_seq; ++s)
    tiles += (L.cu_seqlens_q_host[s + 1] - L.cu_seqlens_q_host[s] + ra::kFwdBlockM - 1) /
             ra::kFwdBlockM;
  const long long wg = tiles * L.hq;
  if (wg <= 0) return 1;
  if (wg < 256) return (int)std::min<long long>(8, (512 + wg - 1) / wg);
  // Long shares of 1-4 workgroups per slot (two per CU): rows on average
  // seeing 64K keys or more make the float32 partials a small cost (0.3% of
  // a 256K MLA share), while halving every unit shortens the tail of the
  // two-round schedule: that share gains 1.3% (1065 -> 1080 TFLOP/s).  The
  // 32K GQA share (16K keys per row) loses 5.5% split, so it is not.
  if (wg < 2048) {
    double rows = 0.0, keys = 0.0;  // visible keys per row ~ half the global document
    for (int s = 0; s < L.n_seq; ++s) {
      const double lq = (double)(L.cu_seqlens_q_host[s + 1] - L.cu_seqlens_q_host[s]);
      rows += lq;
      keys += lq * lq * d->cp_size / 2.0;
    }
    if (rows > 0.0 && keys >= 65536.0 * rows) return 2;
  }
  return 1;
}

// 64-key tiles visited over the ring's blocks by query tile qt (bm rows) of
// a local segment of len rows (nh first-chunk tiles if half tiles): the
// owner's own block up to the tile's last row, an earlier owner's first
// key half, a later owner's whole block if the tile holds second-half rows.
static long long tile_walk(int len, int qt, int nh, int bm, bool half_tiles, int C, int rank) {
  const int half = len / 2;
  long long q0 = (long long)qt * bm, t_hi = len;
  if (half_tiles) {
    if (qt < nh) t_hi = half;
    else q0 = half + (long long)(qt - nh) * bm;
  }
  const long long last = std::min(q0 + bm, t_hi) - 1;
  long long w = 0;
  for (int o = 0; o < C; ++o) {
    const int owner = (rank - o + C) % C;
    long long kend;
    if (o == 0) kend = std::min<long long>(len, last + 1);
    else if (owner < rank) kend = half;
    else kend = last >= half ? len : 0;
    w += (kend + 63) / 64;
  }
  return w;
}

// Per-tile parts for a single sequence split for its size.  A uniform split
// gives every query tile the same number of parts, but the tiles' walks
// differ up to ~60x (second-half rows of early ranks see every later
// owner's whole block), and the launch is one round of workgroups: its
// length is the heaviest tile's part.  With per-tile parts the same number
// of workgroups (split x tiles) is dealt by the tiles' walks (greedy: the
// next part goes to the tile with the longest part), at most `slots` parts
// per tile; parts are taken heaviest first.  Returns the number of partial
// slots (0: the share keeps the uniform split).  RA_FWD_VAR_SPLIT=0 in the
// environment keeps it uniform.
constexpr int kVarSplitSlots = 6;
static int fwd_var_slots(const ra_rank_desc* d, int split) {
  const ra_attn_desc& L = d->local;
  if (split <= 1 || split > 8 || L.n_seq != 1) return 0;
  const char* e = std::getenv("RA_FWD_VAR_SPLIT");
  if (e && !std::strcmp(e, "0")) return 0;
  const long long tiles =
      (L.cu_seqlens_q_host[1] - L.cu_seqlens_q_host[0] + ra::kFwdBlockM - 1) / ra::kFwdBlockM;
  if (tiles <= 0 || tiles * split > ra::kMaxTileOrder) return 0;
  // the size rule's small shares (or a forced split)
  const char* f = std::getenv("RA_FWD_KV_SPLIT");
  if (!(f && *f) && tiles * L.hq >= 256) return 0;
  return std::max(split, kVarSplitSlots);
}

// Deals `total` workgroups over tiles of walk lengths w (at least one per
// tile, at most `cap`, never more than a tile's walk): each next part goes
// to the tile whose parts are longest.  Writes the units, heaviest part
// first, into rk->tile_order as (tile << 6 | part << 3 | parts - 1), sets
// rk->var_split and returns the number of units; parts[t] (if given)
// receives each tile's part count.
static int plan_tile_parts(const std::vector<long long>& w, long long total, int cap,
                           ra::RankKV* rk, uint8_t* parts_out) {
  const int nt = (int)w.size();
  std::vector<int> parts(nt, 1);
  for (long long n = nt; n < total; ++n) {
    int best = -1;
    for (int t = 0; t < nt; ++t)
      if (parts[t] < cap && parts[t] < w[t] &&
          (best < 0 || (w[t] + parts[t] - 1) / parts[t] > (w[best] + parts[best] - 1) / parts[best]))
        best = t;
    if (best < 0) break;
    ++parts[best];
  }
  std::vector<std::pair<long long, int>> units;  // (part length, entry)
  for (int t = 0; t < nt; ++t) {
    if (parts_out) parts_out[t] = (uint8_t)parts[t];
    for (int q = 0; q < parts[t]; ++q)
      units.emplace_back((w[t] - q + parts[t] - 1) / parts[t], (t << 6) | (q << 3) | (parts[t] - 1));
  }
  std::stable_sort(units.begin(), units.end(),
                   [](const std::pair<long long, int>& x, const std::pair<long long, int>& y) {
                     return x.first > y.first;
                   });
  for (size_t u = 0; u < units.size(); ++u) rk->tile_order[u] = (uint16_t)units[u].second;
  rk->var_split = 1;
  return (int)units.size();
}

// Walk lengths of a single sequence's 128-row query tiles in a rank share
// (the 4-wave forward's and the dQ kernel's tile height).
static_assert(ra::kFwdBlockM == 128, "128-row query tiles");
static std::vector<long long> single_walks(const ra_attn_desc& L, int C, int rank) {
  const int len = L.cu_seqlens_q_host[1] - L.cu_seqlens_q_host[0];
  const int nt = (len + 127) / 128;
  std::vector<long long> w(nt);
  for (int t = 0; t < nt; ++t) w[t] = tile_walk(len, t, 0, 128, false, C, rank);
  return w;
}

// Half tiles (ping-pong kernel, fused rank share of packed documents):
// tile each zig-zag chunk of a document on its own.  A 256-row tile that
// straddles a document's two chunks runs the later owners' blocks, which
// only the second chunk sees, with its first-chunk waves idle; separate
// tiles skip those blocks whole, at the price of more padding.  So they pay
// off on ranks that have later owners (rank < C - 1): on the 128K mix at
// CP 16 ranks 0-13 ran 4-8% faster, rank 14 the same, rank 15 1-3% slower,
// the step 530 -> 563 TFLOP/s with them on every rank.  A single sequence
// splits into whole tiles either way.  RA_FWD_HALF_TILES=0/1 in the
// environment forces the choice.
static bool fwd_half_tiles(const ra_rank_desc* d) {
  const char* e = std::getenv("RA_FWD_HALF_TILES");
  if (e && !std::strcmp(e, "1")) return true;
  if (e && !std::strcmp(e, "0")) return false;
  return d->local.n_seq > 1 && d->rank < d->cp_size - 1;
}

ra_status ra_rank_forward_workspace(const ra_rank_desc* d, size_t* bytes) {
  if (!d || !bytes) return fail(RA_ERR_INVALID_ARG, "NULL argument");
  Checked c;
  ra_status st = check_rank_common(d->local, d->cp_size, d->rank, d->k_blocks, d->v_blocks, &c);
  if (st != RA_OK) return st;
  const size_t out_b = align256((size_t)c.total_q * d->local.hq * d->local.dv * sizeof(float));
  const size_t lse_b = align256((size_t)c.total_q * d->local.hq * sizeof(float));
  size_t b = 0;
  if (d->fuse_merge == 2 && d->local.dtype == RA_BF16) {
    // one launch writing the output directly, or with a KV split the
    // float32 partials of every part
    const int split = fwd_kv_split(d, c);
    const int slots = fwd_var_slots(d, split);
    *bytes = split > 1 ? (size_t)(slots ? slots : split) * (out_b + lse_b) : 0;
    return ok();
  }
  if (d->out_dtype != RA_FP32) b += out_b;                   // fp32 accumulator
  if (!d->fuse_merge && d->cp_size > 1) b += out_b + lse_b;  // one partial
  *bytes = b;
  return ok();
}

// Query tiles (bm rows) of a packed rank share: their number, and the order
// in which the launch takes them.  The work of a tile is estimated by the
// 64-key tiles it visits over the ring's blocks (the kernel's block walk);
// heaviest first is the longest-processing-time order, so a launch over
// many short documents and a few long ones does not end on a long
// document's tiles.  The tile list is segment by segment, each segment's
// heaviest (last) tile first.  Up to kMaxTileOrder tiles the order is by
// tile (tile_ordered = 1); beyond, up to kMaxTileOrder segments, by segment,
// each ranked by its heaviest tile (tile_ordered = 2); beyond that the list
// order stands.
static ra_status order_packed_tiles(const ra_attn_desc& L, int C, int rank, int bm,
                                     bool half_tiles, ra::RankKV* rk, int32_t* n_tiles) {
  std::vector<std::pair<long long, int>> cost, seg_cost;  // (estimated work, tile or segment)
  long long n = 0;
  for (int s = 0; s < L.n_seq; ++s) {
    const int len = L.cu_seqlens_q_host[s + 1] - L.cu_seqlens_q_host[s], half = len / 2;
    const int nh = half_tiles ? (half + bm - 1) / bm : 0;
    const int nt = half_tiles ? nh + (len - half + bm - 1) / bm : (len + bm - 1) / bm;
    long long heaviest = 0;
    for (int i = 0; i < nt; ++i, ++n) {
      const long long w = tile_walk(len, nt - 1 - i, nh, bm, half_tiles, C, rank);
      if (n < ra::kMaxTileOrder) cost.emplace_back(w, (int)n);
      heaviest = std::max(heaviest, w);
    }
    if (s < ra::kMaxTileOrder) seg_cost.emplace_back(heaviest, s);
  }
  if (n * L.hq > 0x7fffffffLL) return fail(RA_ERR_UNSUPPORTED, "too many query tiles");
  *n_tiles = (int32_t)n;
  auto by_cost = [](const std::pair<long long, int>& x, const std::pair<long long, int>& y) {
    return x.first > y.first;
  };
  rk->tile_ordered = 0;
  if (n <= ra::kMaxTileOrder) {
    rk->tile_ordered = 1;
    std::stable_sort(cost.begin(), cost.end(), by_cost);
    for (int u = 0; u < (int)n; ++u) rk->tile_order[u] = (uint16_t)cost[u].second;
  } else if (L.n_seq <= ra::kMaxTileOrder) {
    rk->tile_ordered = 2;
    std::stable_sort(seg_cost.begin(), seg_cost.end(), by_cost);
    for (int u = 0; u < L.n_seq; ++u) rk->tile_order[u] = (uint16_t)seg_cost[u].second;
  }
  return RA_OK;
}

ra_status ra_rank_forward(const ra_rank_desc* d, void* stream) {
  if (!d) return fail(RA_ERR_INVALID_ARG, "descriptor is NULL");
  hipStream_t hs = (hipStream_t)stream;
  Checked c;
  ra_status st = check_rank_common(d->local, d->cp_size, d->rank, d->k_blocks, d->v_blocks, &c);
  if (st != RA_OK) return st;
  if (!d->out || !d->lse) return fail(RA_ERR_INVALID_ARG, "out or lse is NULL");
  if (d->out_dtype != RA_BF16 && d->out_dtype != RA_FP32)
    return fail(RA_ERR_INVALID_ARG, "unknown out_dtype");
  if (!aligned16(d->out)) return fail(RA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  size_t need = 0;
  if ((st = ra_rank_forward_workspace(d, &need)) != RA_OK) return st;
  if (need && (!d->workspace || d->workspace_bytes < need))
    return fail(RA_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", d->workspace_bytes,
                need);
  if (need && !aligned16(d->workspace))
    return fail(RA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const ra_attn_desc& L = d->local;
  hipError_t e;
  if (d->fuse_merge == 2 && L.dtype == RA_BF16) {
    // the whole share in one launch: every owner's block in ring order,
    // merged in registers, final output written by the epilogue
    if (d->cp_size > ra::kMaxCp)
      return fail(RA_ERR_UNSUPPORTED, "fused rank forward supports cp_size <= %d", ra::kMaxCp);
    ra::RankKV rk;
    std::memset(&rk, 0, sizeof(rk));
    rk.cp = d->cp_size;
    rk.rank = d->rank;
    for (int j = 0; j < d->cp_size; ++j) {
      rk.k[j] = d->k_blocks[j];
      rk.v[j] = d->v_blocks[j];
    }
    ra_attn_desc sd = L;
    sd.k = d->k_blocks[0];
    sd.v = d->v_blocks[0];
    sd.causal = 1;
    sd.q_part = RA_PART_ALL;
    sd.k_part = RA_PART_ALL;
    Checked cs;
    if ((st = check_desc(&sd, true, &cs)) != RA_OK) return st;
    ra::AttnArgs a = make_args(&sd, cs);
    a.out = static_cast<float*>(d->out);
    a.lse = d->lse;
    int split = fwd_kv_split(d, c);
    const int slots = fwd_var_slots(d, split);
    if (slots) {
      const std::vector<long long> w = single_walks(L, d->cp_size, d->rank);
      rk.fwd_tiles = plan_tile_parts(w, (long long)split * (long long)w.size(), slots, &rk, nullptr);
      split = slots;  // partial slots; unused ones get lse = -inf from the tile's part 0
    }
    rk.split = split;
    const size_t out_b = align256((size_t)c.total_q * L.hq * L.dv * sizeof(float));
    const size_t lse_b = align256((size_t)c.total_q * L.hq * sizeof(float));
    if (split > 1) {
      // parts: split float32 outputs, then split lse arrays
      rk.part_out_stride = (int64_t)(out_b / sizeof(float));
      rk.part_lse_stride = (int64_t)(lse_b / sizeof(float));
      a.out = static_cast<float*>(d->workspace);
      a.lse = reinterpret_cast<float*>(static_cast<char*>(d->workspace) + split * out_b);
    }
    const bool pp = use_pingpong(&L, RA_PART_ALL);
    if (pp && fwd_half_tiles(d)) {
      // tiles of the first chunk (len/2 rows) plus those of the second
      // (len - len/2 rows; one more than the first when a cp_size = 1
      // share has an odd length)
      int nh = 0;
      for (int s = 0; s < L.n_seq; ++s) {
        const int len = L.cu_seqlens_q_host[s + 1] - L.cu_seqlens_q_host[s];
        const int half = len / 2;
        nh = std::max(nh, (half + 255) / 256 + (len - half + 255) / 256);
      }
      a.half_tiles = 1;
      a.n_qtiles_half = nh;
    }
    if (L.n_seq > 1 &&
        (st = order_packed_tiles(L, d->cp_size, d->rank, pp ? 256 : ra::kFwdBlockM,
                                 a.half_tiles != 0, &rk, &rk.fwd_tiles)) != RA_OK)
      return st;
    if (d->events && d->events[0] &&
        (e = hipEventRecord((hipEvent_t)d->events[0], hs)) != hipSuccess)
      return hip_fail(e, "event record");
    if (a.n_qtiles > 0) {
      e = pp
              ? ra::launch_rank_fwd_pp(a, rk, L.dqk, L.dv, d->out_dtype == RA_BF16, hs)
              : ra::launch_rank_fwd_bf16(a, rk, L.dqk, L.dv,
                                         split == 1 && d->out_dtype == RA_BF16, hs);
      if (e != hipSuccess) return hip_fail(e, "rank forward launch");
      if (split > 1) {
        e = ra::launch_split_combine(a.out, a.lse, split, rk.part_out_stride,
                                     rk.part_lse_stride, d->out, d->out_dtype, d->lse,
                                     c.total_q, L.hq, L.dv, hs);
        if (e != hipSuccess) return hip_fail(e, "split combine launch");
      }
    }
    if (d->events && d->events[1] &&
        (e = hipEventRecord((hipEvent_t)d->events[1], hs)) != hipSuccess)
      return hip_fail(e, "event record");
    return ok();
  }
  const size_t out_b = align256((size_t)c.total_q * L.hq * L.dv * sizeof(float));
  char* ws = static_cast<char*>(d->workspace);
  float* acc = nullptr;
  if (d->out_dtype == RA_FP32) {
    acc = static_cast<float*>(d->out);
  } else {
    acc = reinterpret_cast<float*>(ws);
    ws += out_b;
  }
  float* part_out = nullptr;
  float* part_lse = nullptr;
  if (!d->fuse_merge && d->cp_size > 1) {
    part_out = reinterpret_cast<float*>(ws);
    ws += out_b;
    part_lse = reinterpret_cast<float*>(ws);
  }
  for (int s = 0; s < d->cp_size; ++s) {
    const Step p = plan_step(d->rank, s, d->cp_size);
    ra_attn_desc sd = L;
    sd.k = d->k_blocks[p.owner];
    sd.v = d->v_blocks[p.owner];
    sd.causal = p.causal;
    sd.q_part = p.q_part;
    sd.k_part = p.k_part;
    Checked cs;
    if ((st = check_desc(&sd, true, &cs)) != RA_OK) return st;
    if (d->events && d->events[2 * s] &&
        (e = hipEventRecord((hipEvent_t)d->events[2 * s], hs)) != hipSuccess)
      return hip_fail(e, "event record");
    if (s == 0) {
      st = launch_fwd(&sd, cs, acc, d->lse, false, hs);  // the diagonal starts the result
    } else if (d->fuse_merge) {
      st = launch_fwd(&sd, cs, acc, d->lse, true, hs);
    } else {
      st = launch_fwd(&sd, cs, part_out, part_lse, false, hs);
    }
    if (st != RA_OK) return st;
    if (d->events && d->events[2 * s + 1] &&
        (e = hipEventRecord((hipEvent_t)d->events[2 * s + 1], hs)) != hipSuccess)
      return hip_fail(e, "event record");
    if (s > 0 && !d->fuse_merge) {
      e = ra::launch_lse_merge(acc, d->lse, part_out, part_lse, c.total_q, L.hq, L.dv, L.n_seq,
                               L.cu_seqlens_q, p.q_part, cs.max_q_part, hs);
      if (e != hipSuccess) return hip_fail(e, "lse merge launch");
    }
  }
  if (d->out_dtype == RA_BF16) {
    e = ra::launch_cast_f32_bf16(acc, d->out, (int64_t)c.total_q * L.hq * L.dv, hs);
    if (e != hipSuccess) return hip_fail(e, "cast launch");
  }
  return ok();
}

ra_status ra_attn_bwd_delta(const void* out, ra_dtype out_dtype, const void* dout,
                            ra_dtype dout_dtype, int32_t total_t, int32_t hq, int32_t dv,
                            float* delta, void* stream) {
  if (!out || !dout || !delta) return fail(RA_ERR_INVALID_ARG, "NULL buffer");
  if ((out_dtype != RA_BF16 && out_dtype != RA_FP32) ||
      (dout_dtype != RA_BF16 && dout_dtype != RA_FP32))
    return fail(RA_ERR_INVALID_ARG, "unknown dtype");
  if (total_t < 0 || hq <= 0 || dv <= 0) return fail(RA_ERR_INVALID_ARG, "bad sizes");
  hipError_t e = ra::launch_bwd_delta(out, out_dtype, dout, dout_dtype, total_t, hq, dv, delta,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "delta launch");
  return ok();
}

// dK/dV workgroups: 128 keys each, or (d_qk = 128) 32 keys with the query
// iterations split over the workgroup's waves when 128-key workgroups would
// not give every CU one (history blocks of GQA/MHA rank shares).
// RA_BWD_KV_SPLIT=0 or =1 in the environment forces one.
static bool bwd_kv_split(const ra_attn_desc* d, const ra::AttnArgs& a) {
  if (d->dqk != 128) return false;
  const char* e = std::getenv("RA_BWD_KV_SPLIT");
  if (e && !std::strcmp(e, "1")) return true;
  if (e && !std::strcmp(e, "0")) return false;
  return (long long)a.n_seq * a.hkv * a.n_ktiles < 256;
}

// dK/dV query split of a rank-backward step (the workspace holds the
// partials): workgroups of 128 keys, shared by up to kMaxQsplit workgroups
// that each take a contiguous share of the key tile's query iterations.
// Split until the launch has 256 workgroups (one per CU), and at least in
// two on a causal block of fewer than 512 workgroups, whose first key tiles
// see every query and the last ones only a few (with more workgroups than
// that the heavy-first order already evens the CUs out: the 256K MLA
// diagonal block, 1024 workgroups, took the same time split).
// RA_BWD_QSPLIT=n in the environment forces n.
constexpr int kMaxQsplit = 4;
static int bwd_qsplit(const ra_attn_desc* d, const Checked& c) {
  const char* e = std::getenv("RA_BWD_QSPLIT");
  if (e && *e) return std::max(1, std::min(std::atoi(e), kMaxQsplit));
  const long long wg = (long long)d->n_seq * d->hkv * ((c.max_k_part + 127) / 128);
  int n = 1;
  while (n < kMaxQsplit && wg * n < 256) n *= 2;
  if (d->causal && n < 2 && wg < 512) n = 2;
  return n;
}

// Bytes of one query share's dK/dV partial: every key row of the block.
static size_t bwd_part_bytes(const ra_attn_desc* d, const Checked& c) {
  return align256((size_t)c.total_k * d->hkv * (d->dqk + d->dv) * sizeof(float));
}

// dQ key split of a rank-backward step: query tiles of 128 rows shared by up
// to kMaxQsplit workgroups that deal its key tiles among themselves, doubled
// until the dQ launch has 256 workgroups (small shares: an 8K MHA rank's
// history block gives 64-128).  RA_BWD_KSPLIT=n in the environment forces n.
static int bwd_ksplit(const ra_attn_desc* d, const Checked& c) {
  const char* e = std::getenv("RA_BWD_KSPLIT");
  if (e && *e) return std::max(1, std::min(std::atoi(e), kMaxQsplit));
  const long long wg = (long long)d->n_seq * d->hq * ((c.max_q_part + 127) / 128);
  int n = 1;
  while (n < kMaxQsplit && wg * n < 256) n *= 2;
  return n;
}

// Bytes of one key share's dQ partial: every query row of the block.
static size_t bwd_dq_part_bytes(const ra_attn_desc* d, const Checked& c) {
  return align256((size_t)c.total_q * d->hq * d->dqk * sizeof(float));
}

// Workspace bytes past delta that a step needs: its dK/dV partials, then
// its dQ partials.
static size_t bwd_step_parts(const ra_attn_desc* d, const Checked& c) {
  return (size_t)(bwd_qsplit(d, c) - 1) * bwd_part_bytes(d, c) +
         (size_t)(bwd_ksplit(d, c) - 1) * bwd_dq_part_bytes(d, c);
}

static ra_status launch_bwd(const ra_attn_desc* d, const Checked& c, const void* dout,
                            const float* lse, const float* delta, float* dq, float* dk, float* dv,
                            hipStream_t st, int qsplit = 1, float* part = nullptr,
                            int ksplit = 1, float* dq_part = nullptr) {
  ra::AttnArgs a = make_args(d, c);
  a.n_ktiles = (c.max_k_part + 127) / 128;  // 128-key tiles of the dK/dV kernel
  a.dout = dout;
  a.lse_in = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.qsplit = part ? qsplit : 1;
  a.part_keys = c.total_k;
  a.dk_part = part;
  a.dv_part = part ? part + (size_t)(qsplit - 1) * c.total_k * d->hkv * d->dqk : nullptr;
  a.ksplit = dq_part ? ksplit : 1;
  a.dq_part = dq_part;
  // the query-split-over-waves form only where no workspace split runs
  const bool kv_split = a.qsplit == 1 && bwd_kv_split(d, a);
  hipError_t e =
      ra::launch_attn_bwd_bf16(a, d->dqk, d->dv, d->causal != 0, kv_split, c.total_k, st);
  if (e == hipErrorInvalidValue) return fail(RA_ERR_UNSUPPORTED, "backward variant not built");
  if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  return RA_OK;
}

static ra_status check_bwd_extra(const ra_attn_desc* d, const void* dout, const float* lse,
                                 const float* delta, const float* dq, const float* dk,
                                 const float* dv) {
  if (!dout || !lse || !delta || !dq || !dk || !dv)
    return fail(RA_ERR_INVALID_ARG, "NULL buffer");
  if (d->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "backward is bf16 only");
  if (!((d->dqk == 128 && d->dv == 128) || (d->dqk == 192 && d->dv == 128)))
    return fail(RA_ERR_UNSUPPORTED, "backward (dqk, dv) = (%d, %d) not built", d->dqk, d->dv);
  if (d->q_stride_tok && d->q_stride_tok != (int64_t)d->hq * d->dqk)
    return fail(RA_ERR_UNSUPPORTED, "backward needs packed q (dq shares its layout)");
  if (d->k_stride_tok && d->k_stride_tok != (int64_t)d->hkv * d->dqk)
    return fail(RA_ERR_UNSUPPORTED, "backward needs packed k");
  if (d->v_stride_tok && d->v_stride_tok != (int64_t)d->hkv * d->dv)
    return fail(RA_ERR_UNSUPPORTED, "backward needs packed v");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(RA_ERR_INVALID_ARG, "backward buffers must be 16-byte aligned");
  return RA_OK;
}

ra_status ra_block_attn_bwd(const ra_attn_desc* d, const void* dout, const float* lse,
                            const float* delta, float* dq_acc, float* dk_acc, float* dv_acc,
                            void* stream) {
  Checked c;
  ra_status st = check_desc(d, true, &c);
  if (st != RA_OK) return st;
  if ((st = check_bwd_extra(d, dout, lse, delta, dq_acc, dk_acc, dv_acc)) != RA_OK) return st;
  st = launch_bwd(d, c, dout, lse, delta, dq_acc, dk_acc, dv_acc, (hipStream_t)stream);
  return st == RA_OK ? ok() : st;
}

// Step s of a rank backward as a block descriptor (plan of the ring step).
static ra_status rank_bwd_step(const ra_rank_bwd_desc* d, int s, ra_attn_desc* sd, Checked* cs,
                               int* owner) {
  const Step p = plan_step(d->rank, s, d->cp_size);
  *sd = d->local;
  sd->k = d->k_blocks[p.owner];
  sd->v = d->v_blocks[p.owner];
  sd->causal = p.causal;
  sd->q_part = p.q_part;
  sd->k_part = p.k_part;
  *owner = p.owner;
  return check_desc(sd, true, cs);
}

// Rank-fused backward: one dK/dV launch over every owner's key tiles and
// one dQ launch whose query tiles walk all owners' blocks, instead of one
// pair of launches per ring step.  With the dK/dV launch ordered by kv head
// (each XCD's workgroups share that head's Q/dO tiles in its L2) it is the
// faster form on every workload: 8K MHA 306 vs 217 TFLOP/s, 128K varlen 197
// vs 140, 32K GQA 610 vs 597, 256K MLA 660 vs 641 (same box, alternating).
// It also needs no per-step partials: its workspace is delta and, on shares
// with few query tiles, the dQ key-split partials.
// RA_BWD_RANK_FUSED=0 in the environment selects the per-step form.
static bool bwd_rank_fused() {
  const char* e = std::getenv("RA_BWD_RANK_FUSED");
  return !(e && !std::strcmp(e, "0"));
}

// dQ key split of the rank-fused backward: the walk's key tiles of a query
// tile dealt over up to kMaxQsplit workgroups, doubled until the launch has
// 256 workgroups (the dK/dV launch over all owners is large enough alone).
// RA_BWD_KSPLIT=n in the environment forces n.
// 128-row query tiles of the local rows, segment by segment
static long long rank_q_tiles(const ra_attn_desc& L) {
  long long t = 0;
  for (int s = 0; s < L.n_seq; ++s)
    t += (L.cu_seqlens_q_host[s + 1] - L.cu_seqlens_q_host[s] + 127) / 128;
  return t;
}

static int bwd_rank_ksplit(const ra_attn_desc& L, const Checked& c) {
  (void)c;
  const char* e = std::getenv("RA_BWD_KSPLIT");
  if (e && *e) return std::max(1, std::min(std::atoi(e), kMaxQsplit));
  const long long wg = rank_q_tiles(L) * L.hq;
  int n = 1;
  while (n < kMaxQsplit && wg * n < 256) n *= 2;
  return n;
}

// Per-tile key shares of a single sequence's rank-fused dQ launch: as the
// forward's per-tile parts, the ksplit x tiles workgroups are dealt over
// the query tiles by the length of their walks (at most 6 shares per
// tile, or ksplit if larger), since the tiles' walks differ up to ~60x.
// Returns the number of share slots (0: uniform shares).
// RA_BWD_VAR_SPLIT=0 in the environment keeps the shares uniform.
static int bwd_var_slots(const ra_attn_desc& L, int ksplit) {
  if (ksplit <= 1 || L.n_seq != 1) return 0;
  const char* e = std::getenv("RA_BWD_VAR_SPLIT");
  if (e && !std::strcmp(e, "0")) return 0;
  if (rank_q_tiles(L) * ksplit > ra::kMaxTileOrder) return 0;
  return std::max(ksplit, 6);
}

// Workspace: delta [hq, total_q], then
//  - rank-fused: the dQ partials of key shares 1 .. ksplit-1 (of share
//    slots 1 .. slots-1 with per-tile shares);
//  - per step: the dK/dV partials of query shares 1 .. qsplit-1 (and dQ
//    partials) of the step kind that splits most.  Every kind a rank of the
//    ring can meet is counted (the diagonal block, an earlier and a later
//    owner's block), so one workspace serves every rank.
ra_status ra_rank_backward_workspace(const ra_rank_bwd_desc* d, size_t* bytes) {
  if (!d || !bytes) return fail(RA_ERR_INVALID_ARG, "NULL argument");
  Checked c;
  ra_status st = check_rank_common(d->local, d->cp_size, d->rank, d->k_blocks, d->v_blocks, &c);
  if (st != RA_OK) return st;
  const size_t delta_b = align256((size_t)c.total_q * d->local.hq * sizeof(float));
  if (bwd_rank_fused()) {
    const size_t part = align256((size_t)c.total_q * d->local.hq * d->local.dqk * sizeof(float));
    const int ksplit = bwd_rank_ksplit(d->local, c);
    const int slots = bwd_var_slots(d->local, ksplit);
    *bytes = delta_b + (size_t)((slots ? slots : ksplit) - 1) * part;
    return ok();
  }
  size_t parts = 0;
  const int n_kinds = d->cp_size > 1 ? 3 : 1;
  for (int kind = 0; kind < n_kinds; ++kind) {
    // the plan of rank 0 (s = 0), of the last rank at s = 1 (owner before
    // it) and of rank 0 at s = 1 (owner after it)
    const Step p = kind == 0 ? plan_step(0, 0, d->cp_size)
                             : plan_step(kind == 1 ? d->cp_size - 1 : 0, 1, d->cp_size);
    ra_attn_desc sd = d->local;
    sd.k = d->k_blocks[0];
    sd.v = d->v_blocks[0];
    sd.causal = p.causal;
    sd.q_part = p.q_part;
    sd.k_part = p.k_part;
    Checked cs;
    if ((st = check_desc(&sd, true, &cs)) != RA_OK) return st;
    parts = std::max(parts, bwd_step_parts(&sd, cs));
  }
  *bytes = delta_b + parts;
  return ok();
}

ra_status ra_rank_backward(const ra_rank_bwd_desc* d, void* stream) {
  if (!d) return fail(RA_ERR_INVALID_ARG, "descriptor is NULL");
  hipStream_t hs = (hipStream_t)stream;
  Checked c;
  ra_status st = check_rank_common(d->local, d->cp_size, d->rank, d->k_blocks, d->v_blocks, &c);
  if (st != RA_OK) return st;
  if (!d->out || !d->dout || !d->lse || !d->dq || !d->dk_blocks || !d->dv_blocks)
    return fail(RA_ERR_INVALID_ARG, "NULL buffer");
  if (d->out_dtype != RA_BF16 && d->out_dtype != RA_FP32)
    return fail(RA_ERR_INVALID_ARG, "unknown out_dtype");
  for (int j = 0; j < d->cp_size; ++j)
    if (!d->dk_blocks[j] || !d->dv_blocks[j])
      return fail(RA_ERR_INVALID_ARG, "gradient block of owner %d is NULL", j);
  size_t need = 0;
  if ((st = ra_rank_backward_workspace(d, &need)) != RA_OK) return st;
  if (!d->workspace || d->workspace_bytes < need)
    return fail(RA_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", d->workspace_bytes,
                need);
  const ra_attn_desc& L = d->local;
  for (int j = 0; j < d->cp_size; ++j) {
    ra_attn_desc t = L;
    t.k = d->k_blocks[j];
    t.v = d->v_blocks[j];
    if ((st = check_bwd_extra(&t, d->dout, d->lse, static_cast<const float*>(d->workspace),
                              d->dq, d->dk_blocks[j], d->dv_blocks[j])) != RA_OK)
      return st;
  }
  float* delta = static_cast<float*>(d->workspace);
  const size_t delta_b = align256((size_t)c.total_q * L.hq * sizeof(float));
  float* part = reinterpret_cast<float*>(static_cast<char*>(d->workspace) + delta_b);
  hipError_t e;
  if (bwd_rank_fused()) {
    if (d->cp_size > ra::kMaxCp)
      return fail(RA_ERR_UNSUPPORTED, "rank-fused backward supports cp_size <= %d", ra::kMaxCp);
    ra::RankKV rk;
    ra::RankGrad rg;
    std::memset(&rk, 0, sizeof(rk));
    std::memset(&rg, 0, sizeof(rg));
    rk.cp = d->cp_size;
    rk.rank = d->rank;
    for (int j = 0; j < d->cp_size; ++j) {
      rk.k[j] = d->k_blocks[j];
      rk.v[j] = d->v_blocks[j];
      rg.dk[j] = d->dk_blocks[j];
      rg.dv[j] = d->dv_blocks[j];
    }
    // live 128-key tiles of each step's block (the dK/dV grid per kv head),
    // with their work in 32-row query iterations (plus two for a
    // workgroup's set-up and epilogue)
    long long kv_tiles = 0;
    std::vector<std::pair<long long, int>> kv_cost;
    for (int o = 0; o < d->cp_size; ++o) {
      rk.kv_tile_off[o] = (int32_t)kv_tiles;
      int causal, qp, kp;
      ra::owner_plan(d->rank, (d->rank - o + d->cp_size) % d->cp_size, &causal, &qp, &kp);
      for (int s = 0; s < L.n_seq; ++s) {
        int ql, qh, kl, kh;
        ra::part_range(L.cu_seqlens_q_host[s], L.cu_seqlens_q_host[s + 1], qp, &ql, &qh);
        ra::part_range(L.cu_seqlens_k_host[s], L.cu_seqlens_k_host[s + 1], kp, &kl, &kh);
        if (qh <= ql || kh <= kl) continue;
        const int nkt = (kh - kl + 127) / 128, nqt = (qh - ql + 31) / 32;
        for (int kt = 0; kt < nkt && kv_tiles + kt < ra::kMaxTileOrder; ++kt)
          kv_cost.emplace_back((long long)std::max(nqt - (causal ? 4 * kt : 0), 0) *
                                       (L.hq / L.hkv) + 2,
                               (int)(kv_tiles + kt));
        kv_tiles += nkt;
      }
      if (kv_tiles * L.hkv > 0x7fffffffLL)
        return fail(RA_ERR_UNSUPPORTED, "rank-fused backward: too many key tiles");
    }
    rk.kv_tile_off[d->cp_size] = (int32_t)kv_tiles;
    // dK/dV: each kv head's key tiles heaviest first where they fit the
    // order (the causal diagonal's tiles shrink along the block, and a
    // workgroup holds a CU for its whole query walk); the dQ launch gets its
    // own copy of the arguments
    ra::RankKV rkq = rk;
    rk.tile_ordered = kv_tiles <= ra::kMaxTileOrder ? 1 : 0;
    if (rk.tile_ordered) {
      std::stable_sort(kv_cost.begin(), kv_cost.end(),
                       [](const std::pair<long long, int>& x, const std::pair<long long, int>& y) {
                         return x.first > y.first;
                       });
      for (size_t u = 0; u < kv_cost.size(); ++u) rk.tile_order[u] = (uint16_t)kv_cost[u].second;
    }
    const long long q_tiles = rank_q_tiles(L);
    if (q_tiles * L.hq * kMaxQsplit > 0x7fffffffLL)
      return fail(RA_ERR_UNSUPPORTED, "rank-fused backward: too many query tiles");
    rkq.q_tiles = (int32_t)q_tiles;
    // the dQ tiles walk the blocks as the forward's do: same heaviest-first
    // order over packed segments (a single sequence's tiles already run
    // heaviest first: last rows first)
    if (L.n_seq > 1 && (st = order_packed_tiles(L, d->cp_size, d->rank, 128, false, &rkq,
                                                &rkq.q_tiles)) != RA_OK)
      return st;
    ra_attn_desc sd = L;
    sd.k = d->k_blocks[0];
    sd.v = d->v_blocks[0];
    sd.causal = 0;
    sd.q_part = RA_PART_ALL;
    sd.k_part = RA_PART_ALL;
    Checked cs;
    if ((st = check_desc(&sd, true, &cs)) != RA_OK) return st;
    ra::AttnArgs a = make_args(&sd, cs);
    a.n_ktiles = (cs.max_k_part + 127) / 128;
    a.dout = d->dout;
    a.lse_in = d->lse;
    a.delta = delta;
    a.dq = d->dq;
    const int ksplit = bwd_rank_ksplit(L, c);
    const int slots = bwd_var_slots(L, ksplit);
    ra::TileShares ts;
    ts.var = 0;
    if (slots) {
      const std::vector<long long> w = single_walks(L, d->cp_size, d->rank);
      rkq.q_tiles = plan_tile_parts(w, (long long)ksplit * (long long)w.size(), slots, &rkq, ts.n);
      ts.var = 1;
    }
    a.ksplit = slots ? slots : ksplit;
    a.dq_part = a.ksplit > 1 ? part : nullptr;
    if (d->events && d->events[0] &&
        (e = hipEventRecord((hipEvent_t)d->events[0], hs)) != hipSuccess)
      return hip_fail(e, "event record");
    e = ra::launch_bwd_delta(d->out, d->out_dtype, d->dout, L.dtype, c.total_q, L.hq, L.dv,
                             delta, hs);
    if (e != hipSuccess) return hip_fail(e, "delta launch");
    if (a.n_qtiles > 0) {
      e = ra::launch_rank_bwd_bf16(a, rk, rkq, rg, ts, L.dqk, L.dv, hs);
      if (e == hipErrorInvalidValue) return fail(RA_ERR_UNSUPPORTED, "backward variant not built");
      if (e != hipSuccess) return hip_fail(e, "rank backward launch");
    }
    void* last = d->events ? d->events[2 * d->cp_size - 1] : nullptr;
    if (last && (e = hipEventRecord((hipEvent_t)last, hs)) != hipSuccess)
      return hip_fail(e, "event record");
    return ok();
  }
  // events[0] goes before delta, so that it marks the rank's first launch
  if (d->events && d->events[0] &&
      (e = hipEventRecord((hipEvent_t)d->events[0], hs)) != hipSuccess)
    return hip_fail(e, "event record");
  e = ra::launch_bwd_delta(d->out, d->out_dtype, d->dout, L.dtype, c.total_q, L.hq, L.dv, delta,
                           hs);
  if (e != hipSuccess) return hip_fail(e, "delta launch");
  for (int s = 0; s < d->cp_size; ++s) {
    ra_attn_desc sd;
    Checked cs;
    int owner;
    if ((st = rank_bwd_step(d, s, &sd, &cs, &owner)) != RA_OK) return st;
    // the partials fit the workspace (sized by ra_rank_backward_workspace)
    const int qsplit = bwd_qsplit(&sd, cs), ksplit = bwd_ksplit(&sd, cs);
    if (bwd_step_parts(&sd, cs) > d->workspace_bytes - delta_b)
      return fail(RA_ERR_INVALID_ARG, "workspace too small for the dK/dV and dQ splits");
    float* dq_part = reinterpret_cast<float*>(reinterpret_cast<char*>(part) +
                                              (size_t)(qsplit - 1) * bwd_part_bytes(&sd, cs));
    if (s > 0 && d->events && d->events[2 * s] &&
        (e = hipEventRecord((hipEvent_t)d->events[2 * s], hs)) != hipSuccess)
      return hip_fail(e, "event record");
    st = launch_bwd(&sd, cs, d->dout, d->lse, delta, d->dq, d->dk_blocks[owner],
                    d->dv_blocks[owner], hs, qsplit, qsplit > 1 ? part : nullptr, ksplit,
                    ksplit > 1 ? dq_part : nullptr);
    if (st != RA_OK) return st;
    if (d->events && d->events[2 * s + 1] &&
        (e = hipEventRecord((hipEvent_t)d->events[2 * s + 1], hs)) != hipSuccess)
      return hip_fail(e, "event record");
  }
  return ok();
}

ra_status ra_shard_tokens(ra_map kind, int32_t cp_size, int32_t rank, int32_t n_seq,
                          const int32_t* cu_seqlens_global, int32_t* tokens, int32_t capacity,
                          int32_t* n_tokens) {
  ra_status st = check_map(kind, cp_size, rank, n_seq, cu_seqlens_global);
  if (st != RA_OK) return st;
  if (!tokens || !n_tokens) return fail(RA_ERR_INVALID_ARG, "NULL output");
  const int64_t T = cu_seqlens_global[n_seq], n = T / cp_size;
  if (capacity < n) return fail(RA_ERR_INVALID_ARG, "capacity %d < %lld tokens", capacity, (long long)n);
  if (kind == RA_MAP_STRIPED) {
    for (int64_t i = 0; i < n; ++i) tokens[i] = (int32_t)(i * cp_size + rank);
  } else {
    for (const Run& x : rank_runs(kind, cp_size, rank, n_seq, cu_seqlens_global))
      for (int64_t i = 0; i < x.len; ++i) tokens[x.local_lo + i] = (int32_t)(x.global_lo + i);
  }
  *n_tokens = (int32_t)n;
  return ok();
}

ra_status ra_step_segments(ra_map kind, int32_t cp_size, int32_t rank, int32_t owner,
                           int32_t n_seq, const int32_t* cu_seqlens_global, ra_segment* segs,
                           int32_t capacity, int32_t* n_segs) {
  ra_status st = check_map(kind, cp_size, rank, n_seq, cu_seqlens_global);
  if (st != RA_OK) return st;
  if (owner < 0 || owner >= cp_size) return fail(RA_ERR_INVALID_ARG, "bad owner %d", owner);
  if (!segs || !n_segs) return fail(RA_ERR_INVALID_ARG, "NULL output");
  std::vector<ra_segment> v;
  if ((st = step_segments(kind, cp_size, rank, owner, n_seq, cu_seqlens_global, &v)) != RA_OK)
    return st;
  if ((int64_t)v.size() > capacity)
    return fail(RA_ERR_INVALID_ARG, "capacity %d < %zu rectangles", capacity, v.size());
  std::copy(v.begin(), v.end(), segs);
  *n_segs = (int32_t)v.size();
  return ok();
}

static ra_status token_copy(const void* src, void* dst, int64_t row_bytes, int32_t n_rows,
                            const int32_t* tok, const int32_t* tok_host, int32_t n, bool gather,
                            void* stream) {
  if (!src || !dst || (n > 0 && (!tok || !tok_host)))
    return fail(RA_ERR_INVALID_ARG, "NULL argument");
  if (row_bytes <= 0 || (row_bytes % 16) || !aligned16(src) || !aligned16(dst))
    return fail(RA_ERR_INVALID_ARG, "rows must be 16-byte multiples and aligned");
  if (n < 0 || n_rows < 0) return fail(RA_ERR_INVALID_ARG, "negative count");
  for (int32_t i = 0; i < n; ++i)
    if (tok_host[i] < 0 || tok_host[i] >= n_rows)
      return fail(RA_ERR_INVALID_ARG, "token %d of row %d outside [0, %d)", tok_host[i], i, n_rows);
  hipError_t e = ra::launch_gather_tokens(src, dst, row_bytes, tok, n, gather, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "token copy launch");
  return ok();
}

ra_status ra_gather_tokens(const void* src, void* dst, int64_t row_bytes, int32_t n_rows,
                           const int32_t* tokens_dev, const int32_t* tokens_host, int32_t n,
                           void* stream) {
  return token_copy(src, dst, row_bytes, n_rows, tokens_dev, tokens_host, n, true, stream);
}

ra_status ra_scatter_tokens(const void* src, void* dst, int64_t row_bytes, int32_t n_rows,
                            const int32_t* tokens_dev, const int32_t* tokens_host, int32_t n,
                            void* stream) {
  return token_copy(src, dst, row_bytes, n_rows, tokens_dev, tokens_host, n, false, stream);
}

static ra_status check_segments(const ra_segment* segs, int32_t n_seg, int64_t Tq, int64_t Tk,
                                int* max_q) {
  if (n_seg < 0) return fail(RA_ERR_INVALID_ARG, "negative n_seg");
  if (n_seg > 0 && !segs) return fail(RA_ERR_INVALID_ARG, "segments are NULL");
  std::vector<std::pair<int32_t, int32_t>> rows;
  *max_q = 0;
  for (int i = 0; i < n_seg; ++i) {
    const ra_segment& g = segs[i];
    if (g.q_lo < 0 || g.q_lo > g.q_hi || g.q_hi > Tq || g.k_lo < 0 || g.k_lo > g.k_hi ||
        g.k_hi > Tk)
      return fail(RA_ERR_INVALID_ARG, "rectangle %d outside the buffers", i);
    if (g.diag < -(1 << 30) || g.diag > (1 << 30))
      return fail(RA_ERR_INVALID_ARG, "rectangle %d: diag out of range", i);
    if (g.q_hi > g.q_lo) rows.push_back({g.q_lo, g.q_hi});
    *max_q = std::max(*max_q, g.q_hi - g.q_lo);
  }
  std::sort(rows.begin(), rows.end());
  for (size_t i = 1; i < rows.size(); ++i)
    if (rows[i].first < rows[i - 1].second)
      return fail(RA_ERR_INVALID_ARG, "rectangles overlap in rows [%d, %d)", rows[i].first,
                  rows[i - 1].second);
  return RA_OK;
}

ra_status ra_block_attn_fwd_segments(const ra_attn_desc* d, int32_t n_seg,
                                     const ra_segment* segs_dev, const ra_segment* segs_host,
                                     float* out, float* lse, int32_t merge, void* stream) {
  if (!d) return fail(RA_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->n_seq != 1)
    return fail(RA_ERR_INVALID_ARG, "rectangle lists take n_seq = 1 (buffer row counts)");
  ra_attn_desc t = *d;
  t.causal = 0;
  t.q_part = RA_PART_ALL;
  t.k_part = RA_PART_ALL;
  Checked c;
  ra_status st = check_desc(&t, true, &c);
  if (st != RA_OK) return st;
  if (d->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "rectangle lists are bf16 only");
  if (!out || !lse) return fail(RA_ERR_INVALID_ARG, "out or lse is NULL");
  if (!aligned16(out)) return fail(RA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (n_seg > 0 && !segs_dev) return fail(RA_ERR_INVALID_ARG, "device segments are NULL");
  int max_q = 0;
  if ((st = check_segments(segs_host, n_seg, c.total_q, c.total_k, &max_q)) != RA_OK) return st;
  if (n_seg == 0 || max_q == 0) return ok();
  ra::AttnArgs a = make_args(&t, c);
  a.segs = segs_dev;
  a.n_seq = n_seg;
  a.n_qtiles = (max_q + ra::kFwdBlockM - 1) / ra::kFwdBlockM;
  a.out = out;
  a.lse = lse;
  hipError_t e = ra::launch_attn_fwd_segments(a, d->dqk, d->dv, merge != 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rectangle attention launch");
  return ok();
}

ra_status ra_segments_work(const ra_segment* segs, int32_t n_seg, int32_t hq,
                           int64_t* visible_pairs, int64_t* tiles_visited, int64_t* tiles_skipped) {
  if (!visible_pairs || !tiles_visited || !tiles_skipped)
    return fail(RA_ERR_INVALID_ARG, "NULL output");
  if (hq <= 0) return fail(RA_ERR_INVALID_ARG, "hq must be >= 1");
  int max_q = 0;
  ra_status st = check_segments(segs, n_seg, INT32_MAX, INT32_MAX, &max_q);
  if (st != RA_OK) return st;
  const int bm = ra::kFwdBlockM, bn = ra::kFwdBlockN;
  int64_t pairs = 0, vis = 0, skip = 0;
  for (int i = 0; i < n_seg; ++i) {
    const ra_segment& g = segs[i];
    const int64_t lq = g.q_hi - g.q_lo, lk = g.k_hi - g.k_lo;
    const bool full = g.diag >= lk;
    for (int64_t r = 0; r < lq; ++r)
      pairs += full ? lk : std::min<int64_t>(lk, std::max<int64_t>(0, r + g.diag + 1));
    const int64_t all_tiles = (lk + bn - 1) / bn;
    for (int64_t q0 = 0; q0 < lq; q0 += bm) {
      const int64_t last = std::min<int64_t>(q0 + bm, lq) - 1;
      const int64_t kend = full ? lk : std::min<int64_t>(lk, std::max<int64_t>(0, last + g.diag + 1));
      const int64_t v = (kend + bn - 1) / bn;
      vis += v;
      skip += all_tiles - v;
    }
  }
  *visible_pairs = pairs * hq;
  *tiles_visited = vis * hq;
  *tiles_skipped = skip * hq;
  return ok();
}

ra_status ra_block_attn_work(const ra_attn_desc* d, int64_t* visible_pairs,
                             int64_t* tiles_visited, int64_t* tiles_skipped) {
  Checked c;
  ra_status st = check_desc(d, false, &c);
  if (st != RA_OK) return st;
  if (!visible_pairs || !tiles_visited || !tiles_skipped)
    return fail(RA_ERR_INVALID_ARG, "NULL output");
  const int bm = d->dtype == RA_BF16 ? ra::kFwdBlockM : ra::kF32BlockM;
  const int bn = d->dtype == RA_BF16 ? ra::kFwdBlockN : ra::kF32BlockN;
  int64_t pairs = 0, vis = 0, skip = 0;
  for (int s = 0; s < d->n_seq; ++s) {
    const int lq = part_len(d->cu_seqlens_q_host[s + 1] - d->cu_seqlens_q_host[s], d->q_part);
    const int lk = part_len(d->cu_seqlens_k_host[s + 1] - d->cu_seqlens_k_host[s], d->k_part);
    if (d->causal)
      for (int i = 0; i < lq; ++i) pairs += std::min(lk, i + 1);
    else
      pairs += (int64_t)lq * lk;
    const int all_tiles = (lk + bn - 1) / bn;
    for (int q0 = 0; q0 < lq; q0 += bm) {
      const int last = std::min(q0 + bm, lq) - 1;
      const int kend = d->causal ? std::min(lk, last + 1) : lk;
      const int v = (kend + bn - 1) / bn;
      vis += v;
      skip += all_tiles - v;
    }
  }
  *visible_pairs = pairs * d->hq;
  *tiles_visited = vis * d->hq;
  *tiles_skipped = skip * d->hq;
  return ok();
}

}  // extern "C"
