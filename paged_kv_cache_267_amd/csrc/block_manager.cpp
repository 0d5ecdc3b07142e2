// block_manager.cpp -- host-side manager of the physical block pool behind the
// block tables the decode kernels read.
//
// What it manages follows the pages: a pool of fixed-size blocks, a request
// taking ceil(n / block_size) of them as its tokens arrive ("vLLM 0.5 deep
// dive: PagedAttention architecture", chenxutan.com, s2.1); a per-request block
// table over non-contiguous physical blocks, with requests that share a prefix
// sharing its blocks ("vLLM deployment and PagedAttention", crazysre.cn, "Core
// concept"; "vLLM 0.7.2 deep dive: PagedAttention v2 with FlashAttention-3",
// jsqmd.com, s2.1); blocks wholly outside a sliding window no longer needed
// (same page, s2.3).
//
// Design: per-block reference counts; a FIFO free list; forks share every
// block of the parent; appending into a shared, partly filled last block first
// copies it (copy-on-write: the caller copies the filled slots on the device);
// a block whose count drops to zero is parked with the caller's epoch (the
// step that last used it) and returns to the free list only when the caller
// reports that epoch completed, so a step still in flight never sees its
// blocks reused.  Not thread-safe: one host thread per manager.
#include <cstdint>
#include <deque>
#include <new>
#include <utility>
#include <vector>

#include "../../include/pa.h"

struct pa_block_manager {
  struct Seq {
    bool live = false;
    int len = 0;                  // tokens
    std::vector<int32_t> blocks;  // -1: released (before a window)
  };
  int num_blocks = 0, block_size = 0;
  std::vector<int32_t> refs;
  std::deque<int32_t> free_list;
  std::vector<std::pair<uint64_t, int32_t>> parked;  // (epoch, block)
  std::vector<Seq> seqs;

  int take() {
    const int b = free_list.front();
    free_list.pop_front();
    refs[b] = 1;
    return b;
  }
  void drop(int b, uint64_t epoch) {
    if (--refs[b] == 0) parked.emplace_back(epoch, b);
  }
  bool valid_seq(int s) const { return s >= 0 && s < (int)seqs.size() && seqs[s].live; }
};

extern "C" {

pa_block_manager* pa_bm_create(int num_blocks, int block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pa_block_manager* m = new (std::nothrow) pa_block_manager;
  if (!m) return nullptr;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->refs.assign(num_blocks, 0);
    for (int b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

int pa_bm_num_free(const pa_block_manager* m) { return m ? (int)m->free_list.size() : -PA_ERR_NULL; }

int pa_bm_new_sequence(pa_block_manager* m, int parent) {
  if (!m) return -PA_ERR_NULL;
  if (parent >= 0 && !m->valid_seq(parent)) return -PA_ERR_SHAPE;
  pa_block_manager::Seq s;
  s.live = true;
  if (parent >= 0) {
    s.len = m->seqs[parent].len;
    s.blocks = m->seqs[parent].blocks;
    for (int32_t b : s.blocks)
      if (b >= 0) ++m->refs[b];
  }
  m->seqs.push_back(std::move(s));
  return (int)m->seqs.size() - 1;
}

int pa_bm_append(pa_block_manager* m, int seq, int num_tokens, int32_t* slot_mapping,
                 int32_t* cow) {
  if (!m || (num_tokens > 0 && !slot_mapping) || !cow) return PA_ERR_NULL;
  if (!m->valid_seq(seq) || num_tokens < 0) return PA_ERR_SHAPE;
  pa_block_manager::Seq& s = m->seqs[seq];
  const int bs = m->block_size;
  cow[0] = cow[1] = -1;
  if (num_tokens == 0) return PA_OK;
  const int fill = s.len % bs;                 // filled slots of the last block
  const bool shared_tail = fill > 0 && s.blocks.back() >= 0 && m->refs[s.blocks.back()] > 1;
  const int need = (s.len + num_tokens + bs - 1) / bs - (s.len + bs - 1) / bs + (shared_tail ? 1 : 0);
  if ((int)m->free_list.size() < need) return PA_ERR_EXHAUSTED;  // nothing changed
  if (shared_tail) {                           // copy-on-write of the partly filled block
    const int old = s.blocks.back();
    const int nb = m->take();
    --m->refs[old];                            // still held by the other sequences
    s.blocks.back() = nb;
    cow[0] = old;
    cow[1] = nb;
  }
  for (int i = 0; i < num_tokens; ++i) {
    const int pos = s.len + i;
    if (pos % bs == 0) s.blocks.push_back(m->take());
    slot_mapping[i] = s.blocks[pos / bs] * bs + pos % bs;
  }
  s.len += num_tokens;
  return PA_OK;
}

int pa_bm_release_before(pa_block_manager* m, int seq, int first_token, uint64_t epoch) {
  if (!m) return -PA_ERR_NULL;
  if (!m->valid_seq(seq) || first_token < 0 || first_token > m->seqs[seq].len)
    return -PA_ERR_SHAPE;
  pa_block_manager::Seq& s = m->seqs[seq];
  const int upto = first_token / m->block_size;  // blocks wholly before first_token
  int n = 0;
  for (int i = 0; i < upto && i < (int)s.blocks.size(); ++i)
    if (s.blocks[i] >= 0) {
      m->drop(s.blocks[i], epoch);
      s.blocks[i] = -1;
      ++n;
    }
  return n;
}

int pa_bm_free_sequence(pa_block_manager* m, int seq, uint64_t epoch) {
  if (!m) return PA_ERR_NULL;
  if (!m->valid_seq(seq)) return PA_ERR_SHAPE;
  pa_block_manager::Seq& s = m->seqs[seq];
  for (int32_t b : s.blocks)
    if (b >= 0) m->drop(b, epoch);
  s.blocks.clear();
  s.len = 0;
  s.live = false;
  return PA_OK;
}

int pa_bm_reclaim(pa_block_manager* m, uint64_t completed_epoch) {
  if (!m) return -PA_ERR_NULL;
  int n = 0;
  std::vector<std::pair<uint64_t, int32_t>> keep;
  for (const auto& e : m->parked) {
    if (e.first <= completed_epoch) {
      m->free_list.push_back(e.second);
      ++n;
    } else {
      keep.push_back(e);
    }
  }
  m->parked.swap(keep);
  return n;
}

int pa_bm_block_table(const pa_block_manager* m, int seq, int32_t* row, int max_blocks) {
  if (!m || !row) return -PA_ERR_NULL;
  if (!m->valid_seq(seq) || max_blocks < 0) return -PA_ERR_SHAPE;
  const std::vector<int32_t>& b = m->seqs[seq].blocks;
  if ((int)b.size() > max_blocks) return -PA_ERR_SHAPE;
  for (int i = 0; i < max_blocks; ++i) row[i] = i < (int)b.size() ? b[i] : -1;
  return (int)b.size();
}

int pa_bm_seq_len(const pa_block_manager* m, int seq) {
  if (!m) return -PA_ERR_NULL;
  return m->valid_seq(seq) ? m->seqs[seq].len : -PA_ERR_SHAPE;
}

int pa_bm_refcount(const pa_block_manager* m, int block) {
  if (!m) return -PA_ERR_NULL;
  return block >= 0 && block < m->num_blocks ? m->refs[block] : -PA_ERR_SHAPE;
}

}  // extern "C"
