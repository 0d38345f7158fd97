"""CLEAR circular-window attention for AMD Instinct MI355X (gfx950)."""
