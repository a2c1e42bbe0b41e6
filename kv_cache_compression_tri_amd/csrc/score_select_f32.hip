// Fused scoring and selection, float32 keys (the bfloat16 ones and the dispatch are in
// score_select.hip).
#define TRI_SCORE_SELECT_F32
#include "score_select.hip"
