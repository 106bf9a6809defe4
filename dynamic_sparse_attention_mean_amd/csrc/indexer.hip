// Indexer token top-k (placeholder until the indexer kernels land).
#include "common.h"
#include "internal.h"

namespace dsa {
bool indexer_supported() { return false; }
bool attn_token_supported() { return false; }
size_t indexer_workspace_bytes(int Nq, int Nk, int Hi, int route_heads) {
  (void)Hi; (void)route_heads;
  return (size_t)Nq * Nk * 4;
}
hipError_t launch_indexer(const IndexerArgs&, void*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace dsa
