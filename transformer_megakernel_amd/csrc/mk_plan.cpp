// Host-side static scheduler.
//
// The Megakernel article (section "Megakernel: a fusion design from scratch") lays
// out every SM's instruction list before runtime, by model structure, with no
// dynamic branching in scheduling, and reuses it for every token.  Here the lists
// are per CU of a gfx950 part: every matrix of the step is cut into contiguous row
// ranges, one per CU, so that each CU streams an equal share of every phase's bytes
// (a phase is one instruction of one layer).  Attention is cut into (KV head, split)
// items whose key ranges are derived from the position on the device, so the same
// plan serves every context length.
//
// Every list is ordered by phase (layer-major, then the article's instruction
// order), and an instruction only consumes results of strictly earlier phases, so
// with all work-groups resident no CU can wait on work queued behind itself.
#include "mk_plan.h"

#include <algorithm>

#include "mk_shapes.h"

namespace {

void split(int n, int parts, int i, int* r0, int* cnt) {
  long a = (long)n * i / parts, b = (long)n * (i + 1) / parts;
  *r0 = (int)a;
  *cnt = (int)(b - a);
}

// Like split, with part i weighted 1 + skew on even XCDs (i % 8 even) and 1 - skew on
// odd ones.
void split_xcd(int n, int parts, int i, double skew, int* r0, int* cnt) {
  auto edge = [&](int k) {   // rows before part k
    double wsum = 0, wk = 0;
    for (int j = 0; j < parts; ++j) {
      const double wj = (j % 8) % 2 == 0 ? 1 + skew : 1 - skew;
      if (j < k) wk += wj;
      wsum += wj;
    }
    return (long)(n * wk / wsum + 0.5);
  };
  const long a = edge(i), b = edge(i + 1);
  *r0 = (int)a;
  *cnt = (int)(b - a);
}

MkInstr mk(int op, int layer) {
  MkInstr x{};
  x.op = op;
  x.layer = layer;
  x.rs = 1;
  return x;
}

}  // namespace

int mk_check_config(const mk_config& c, std::string* why, int* nch) {
  auto bad = [&](const std::string& m) {
    if (why) *why = m;
    return MK_EINVAL;
  };
  if (c.n_layers < 1 || c.hidden < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.ffn < 1 ||
      c.vocab < 1 || c.max_ctx < 1)
    return bad("every dimension must be positive");
  if (!(c.rms_eps >= 0.0f) || !(c.rope_theta > 0.0f)) return bad("rms_eps must be >= 0 and rope_theta > 0");
  int found = 0;
#define MK_MATCH(D, HQ, HKV, HD, F, NCH) \
  if (!found && c.hidden == D && c.n_q_heads == HQ && c.n_kv_heads == HKV && c.head_dim == HD && c.ffn == F) found = NCH;
  MK_SHAPES(MK_MATCH)
#undef MK_MATCH
  if (!found) {
    std::string m = "unsupported shape (hidden, n_q_heads, n_kv_heads, head_dim, ffn) = (" +
                    std::to_string(c.hidden) + ", " + std::to_string(c.n_q_heads) + ", " +
                    std::to_string(c.n_kv_heads) + ", " + std::to_string(c.head_dim) + ", " +
                    std::to_string(c.ffn) + "); compiled:";
#define MK_LIST(D, HQ, HKV, HD, F, NCH) \
  m += " (" + std::to_string(D) + ", " + std::to_string(HQ) + ", " + std::to_string(HKV) + ", " + \
       std::to_string(HD) + ", " + std::to_string(F) + ")";
    MK_SHAPES(MK_LIST)
#undef MK_LIST
    return bad(m);
  }
  if (nch) *nch = found;
  return MK_OK;
}

int mk_build_plan(const mk_config& c, int n_cus, MkPlan* out, std::string* why) {
  int nch = 0;
  int rc = mk_check_config(c, why, &nch);
  if (rc) return rc;
  if (n_cus < 1) {
    if (why) *why = "n_cus must be positive";
    return MK_EINVAL;
  }
  if ((c.hidden + n_cus - 1) / n_cus > MK_MAX_RES_ROWS) {
    if (why) *why = "hidden / n_cus exceeds the 64 residual rows one CU may own";
    return MK_EINVAL;
  }
  MkPlan p;
  p.n_cus = n_cus;
  p.nch = nch;
  p.page_bytes = MK_PAGE_BYTES;
  // The merge of one head's splits polls 16 splits per round; 32 keeps it to two rounds.
  p.s_max = std::max(1, std::min(n_cus / c.n_kv_heads, 32));
  // Fewest cached keys per split.  At head_dim 64 (the matrix-unit attention takes a wave
  // ~0.45 us per 64-key page) two pages: more CUs per KV head at medium contexts (256
  // greedy steps from context 1024: 595 -> 580 us per step).  At head_dim 128 four
  // 32-key pages: 128-key splits there pushed one of the 8B step's appended K/V elements
  // past the fp32 bound of the parity test.
  p.min_chunk = c.head_dim == 64 ? 128 : 256;
  if (p.s_max < c.n_q_heads / c.n_kv_heads) {
    if (why) *why = "too few CUs for one merger per query head of a group";
    return MK_EINVAL;
  }
  const int d = c.hidden, nq = c.n_q_heads * c.head_dim, nqkv = nq + 2 * c.n_kv_heads * c.head_dim;
  p.off.push_back(0);
  for (int cu = 0; cu < n_cus; ++cu) {
    int o0, on, q0, qn, f0, fn, v0, vn;
    split(d, n_cus, cu, &o0, &on);
    split(nqkv, n_cus, cu, &q0, &qn);
    // LM-head rows: 4 % more for CUs on even XCDs, 4 % fewer on odd ones.  In every run
    // the odd XCDs streamed their blocks a few per cent slower (they finished the LM head
    // 2-4 us after the even ones); with this split the slowest CU finishes ~2 us earlier.
    split_xcd(c.vocab, n_cus, cu, n_cus % 8 == 0 ? 0.04 : 0.0, &v0, &vn);
    // Gate/up features are dealt in blocks of fb features, round-robin over the CUs:
    // block b goes to CU b % n_cus.  A CU's first pages then feed the first down chunk,
    // its next pages the second, and so on, so chunk k is complete once every CU has
    // passed its k-th quarter, long before the slowest CU finishes, and the down chunks'
    // staging overlaps the gate/up streaming.  A block is one page's features (fpp), or
    // eight features (a 64-byte line of link words) where that still gives every CU a whole
    // number of blocks per down chunk: each line of SiLU(g)*u words is then written by one
    // CU only.  Feature q of the instruction is r0 + (q / fb) * rs + q % fb (fb a power of
    // two, log2 in the instruction's field a).
    const int fpp = std::max(1, MK_PAGE_BYTES / (4 * d));
    int fb = fpp;
    if (fpp < 8 && (c.ffn / nch) % (n_cus * 8) == 0 && c.ffn % nch == 0) fb = 8;
    const int fblocks = (c.ffn + fb - 1) / fb;
    f0 = cu * fb;
    fn = 0;
    for (int b = cu; b < fblocks; b += n_cus) fn += std::min(fb, c.ffn - b * fb);
    const int fstride = n_cus * fb;
    int fb_log2 = 0;
    while ((1 << fb_log2) < fb) ++fb_log2;
    for (int l = 0; l < c.n_layers; ++l) {
      MkInstr q = mk(MK_OP_QKV, l);
      q.r0 = q0; q.n = qn; q.k0 = 0; q.kn = d;
      p.rec.push_back(q);
      if (cu < c.n_kv_heads * p.s_max) {
        // KV head cu % Hkv, split cu / Hkv: work-groups are dealt to the XCDs round-robin,
        // so at short contexts (split 0 only) the KV heads' items sit on different XCDs
        // instead of all on one.
        MkInstr a = mk(MK_OP_ATTN, l);
        a.a = cu % c.n_kv_heads;
        a.b = cu / c.n_kv_heads;
        p.rec.push_back(a);
      }
      if (on > 0) {
        MkInstr o = mk(MK_OP_O, l);
        o.r0 = o0; o.n = on; o.k0 = 0; o.kn = nq;
        p.rec.push_back(o);
      }
      MkInstr gu = mk(MK_OP_GATEUP, l);
      gu.r0 = f0; gu.n = fn; gu.k0 = 0; gu.kn = d; gu.rs = fstride; gu.a = fb_log2;
      p.rec.push_back(gu);
      if (on > 0) {
        for (int k = 0; k < nch; ++k) {
          MkInstr dn = mk(MK_OP_DOWN, l);
          dn.r0 = o0; dn.n = on; dn.kn = c.ffn / nch; dn.k0 = k * dn.kn; dn.a = k; dn.b = nch;
          p.rec.push_back(dn);
        }
      }
    }
    // LM-head rows: a contiguous block per CU (measured ahead of dealing rows round-robin:
    // the last CU finished 8 us after the median CU instead of 14 us), sized per XCD above.
    MkInstr lm = mk(MK_OP_LMHEAD, c.n_layers);
    lm.r0 = v0; lm.n = vn; lm.k0 = 0; lm.kn = d; lm.rs = 1;
    p.rec.push_back(lm);
    p.off.push_back((int32_t)p.rec.size());
  }
  *out = std::move(p);
  return MK_OK;
}
