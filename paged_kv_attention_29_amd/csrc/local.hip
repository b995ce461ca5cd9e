// pa_local_virtual_batches: host-side rewriting of a batch for chunked local
// attention (vLLM flash_attn.py, v0.9.0.1 docs,
// make_local_attention_virtual_batches).  Positions are cut into chunks of
// attn_chunk_size tokens and a query sees only the keys of its own chunk,
// up to itself.  Each (sequence, chunk holding some of its queries) becomes
// one virtual sequence: its queries are the sequence's queries in that
// chunk (consecutive rows, so the query and output arrays stay as they
// are), its keys run from the chunk start to its last query, and its
// block-table row is the sequence's row from the chunk's first block.  The
// causal prefill over the virtual batch is then the chunked attention.
//
// Plain host C++ (no device code): the inputs are the host copies of the
// batch metadata a serving loop builds before its launches.
#include <cstdint>

#include "launch.h"

namespace pa {

int local_virtual_batches(int chunk, int block_size, const int32_t* qsl, const int32_t* seq_lens,
                          int num_seqs, const int32_t* block_table, int64_t bt_stride,
                          int bt_cols, int32_t* q_local, int32_t* cu_q_local, int32_t* k_local,
                          int32_t* bt_local) {
  const int pages = chunk / block_size;
  int v = 0;
  if (cu_q_local != nullptr) cu_q_local[0] = qsl[0];
  for (int b = 0; b < num_seqs; ++b) {
    const int q_len = qsl[b + 1] - qsl[b];
    const int L = seq_lens[b];
    if (q_len == 0) continue;
    const int first = L - q_len;  // position of the sequence's first query
    const int c_first = first / chunk, c_last = (L - 1) / chunk;
    for (int c = c_first; c <= c_last; ++c, ++v) {
      if (q_local == nullptr) continue;  // counting only (outputs are all NULL then)
      const int start = c * chunk;
      const int lo = first > start ? first : start;             // first query in the chunk
      const int hi = L - 1 < start + chunk - 1 ? L - 1 : start + chunk - 1;  // last one
      q_local[v] = hi - lo + 1;
      cu_q_local[v + 1] = cu_q_local[v] + q_local[v];
      k_local[v] = hi - start + 1;
      const int32_t* row = block_table + (int64_t)b * bt_stride;
      for (int i = 0; i < pages; ++i) {
        int col = start / block_size + i;
        col = col < bt_cols - 1 ? col : bt_cols - 1;
        bt_local[(int64_t)v * pages + i] = row[col];
      }
    }
  }
  return v;
}

}  // namespace pa
